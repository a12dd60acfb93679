// Main stage of the bf16 attention backward for gfx950 (MI355X).
//
// What it computes ("6.1 FlashAttention V1详解", sections 6.1-6.2;
// "FlashAttention v1～v4 完整进化史", v2 part 1 and v4 part 4): for every
// (query, key) pair P = exp(S - L) is recomputed from Q, K and the saved
// log-sum-exp, and
//   dV += P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dK += dS^T Q,
//   dQ += dS K     (scale is applied to dK here and to dQ in the finish pass);
// dQ is summed over key tiles with float32 atomics into the workspace.
//
// Schedule:
//   * one workgroup (4 waves, one per SIMD) per (batch, head, 256-key tile);
//     each wave owns 64 keys (two 32-key blocks); the dK and dV accumulators
//     of those keys (2 x 64 x d floats) stay in the accumulation registers for
//     the whole pass, and V of the wave's keys is held as MFMA operands;
//   * the workgroup's K tile sits in LDS for the whole pass; query tiles of 32
//     rows (Q, dO, L, D) stream through a 3-stage LDS ring, copied from HBM
//     two tiles ahead of use, one barrier per tile;
//   * S = Q K^T and dP = dO V^T are formed with lanes = keys (Q and dO rows
//     read in a permuted order), so the exponentiated P and dS come out in the
//     operand layout of dV = P^T dO and dK = dS^T Q; the other orientation of
//     Q and dO is read straight from the row-major tiles with
//     ds_read_b64_tr_b16;
//   * dS is written to LDS once (transposed, 16-byte writes); dQ of one
//     query tile is formed during the next: each wave takes one 32-column
//     slice of dQ over all 256 keys (lanes = d) and adds it with buffer
//     atomics; query tiles are visited from the last down to the diagonal so
//     that the workgroups of a (batch, head) add to the same dQ rows at the
//     same time and the atomics stay in L2;
//   * fixed-order mode ("FlashAttention v1～v4 完整进化史", v4 part 4: the
//     deterministic backward orders the reduction across workgroups with
//     semaphores): a wave adds its dQ slice to a query tile only after a
//     per-(query tile, slice) counter shows that every earlier key tile has
//     added its own, and bumps the counter once its adds are complete, so
//     the adds to every dQ element happen in ascending key-tile order. A workgroup only waits on key tiles of its own (batch,
//     head) with smaller workgroup ids, which the hardware dispatches first
//     (ids go to the XCDs round-robin and each XCD starts its workgroups in
//     id order; the tiles of a (batch, head) share one XCD); every wait is
//     bounded, and a wait that runs out raises an error flag that turns dq
//     into NaN instead of hanging;
//   * one wave per SIMD means the wave itself must keep the matrix core fed:
//     the products of a tile run in one interleaved stream (S and dP, dV and
//     dK, and dQ of the previously visited tile), operands are read ahead,
//     and the softmax work (P and dS) runs beside the products instead of
//     between them;
//   * rows of the LDS tiles are XOR-swizzled per 16-byte chunk so that both
//     the 16-row reads and the 4-row transposed reads hit distinct banks.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKW = 64;              // keys per wave
constexpr int kBC = kKW * kWaves;    // keys per workgroup
constexpr int kBR = 32;              // query rows per tile
constexpr int kStages = 3;           // query-tile ring depth
static_assert(kBC == kBwdKeyTile && kBR == kBwdRowTile && kWaves == kBwdSlots, "counter layout of the fixed-order dQ");
// Polls of the fixed-order counters a wave may spend in waits over the whole
// kernel before giving up (each poll is a device-scope load plus a short
// sleep: a second or two in all).
constexpr unsigned kSpinLimit = 1u << 20;

#define LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

template <int N>
using IC = std::integral_constant<int, N>;

template <int D>
struct Cfg {
  static constexpr int RB = 2 * D;                   // bytes per row
  static constexpr int CPR = RB / 16;                // 16-byte chunks per row
  static constexpr int K_BYTES = kBC * RB;           // the workgroup's K tile
  static constexpr int QT = kBR * RB;                // one Q or dO tile
  static constexpr int LD = 1024;                    // L (or D) region: one wave-load
  static constexpr int STAGE = 2 * QT + 2 * LD;      // Q, dO, L, D
  static constexpr int DS_BYTES = kBC * kBR * 2;     // dS^T tile [key][q]
  static constexpr int RPL = 1024 / RB;              // rows per 1 KiB wave-load
  static constexpr int K_LOADS = K_BYTES / 1024 / kWaves;
  static constexpr int QT_LOADS = QT / 1024 / kWaves;
  static constexpr int R_LOADS = 2 * QT_LOADS + 1;   // copies per wave per query tile
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static constexpr int NQ = 16;                      // dQ products per dQ-forming wave per tile
  static constexpr int LDS_BYTES = K_BYTES + 2 * DS_BYTES + kStages * STAGE;
  static_assert(QT_LOADS >= 1 && K_LOADS >= 1, "tile split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(R_LOADS + 32 <= 63, "vmcnt range");
};

// Swizzle of 16-byte chunks in rows of Q, dO and K tiles: conflict-free both
// for 16 consecutive rows at one chunk and for 4 consecutive rows x 4 chunks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 tr_read(const unsigned char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS(i16x4, p)));
}
struct Tr4 {
  u32x2 v[4];
};
__device__ __forceinline__ bf16x8 join(u32x2 lo, u32x2 hi) {
  const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Workgroup barrier ordering LDS only (copies to other ring stages stay in
// flight; each wave first waits for its own copies of the tile).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

#define INL __attribute__((always_inline)) __device__

// DET: dQ contributions are added to the accumulator in ascending key-tile
// order (the float32 atomics of each query tile ordered by a counter).
// Grouped K/V heads (a.group > 1): one query head per workgroup with its
// group's K/V head; float32 dK and dV of each query head go to the workspace
// for a fixed-order sum over the group.
// VARLEN: packed variable-length batch, one workgroup per (sequence, query
// head, key tile) with the sequence's rows and length; key tiles past the
// sequence's end exit at once.
template <int D, bool CAUSAL, bool DET, bool VARLEN>
__global__ __launch_bounds__(kThreads, 1) void bwd_bf16_kernel(BwdArgs a) {
  // Device pass only (the host pass needs just the launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char kt_s[C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char ds_s[2 * C::DS_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char rg_s[kStages * C::STAGE];
  auto ring = [&](int st) INL -> unsigned char* { return rg_s + st * C::STAGE; };
  auto dsb = [&](int b) INL -> unsigned char* { return ds_s + b * C::DS_BYTES; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int ts = j16 >> 2, tq = j16 & 3;     // transposed-read source row / column group

  int wg = blockIdx.x;
  // Packed variable-length batch: key tile outermost (all sequences' and
  // heads' tile 0 first, the heaviest of each); with the (sequence, head)
  // pairs a multiple of 8, each pair stays on one XCD (workgroups go to XCDs
  // round-robin by id) and every XCD runs its pairs tile-major. Otherwise the
  // tiles of one (batch, head) are grouped on one XCD, tile 0 first.
  if (a.remap && !VARLEN) wg = xcd_remap(wg, gridDim.x);
  const int nbh = VARLEN ? (int)gridDim.x / a.n_tiles : 0;
  int bhc_, kt_;
  if (VARLEN && a.remap && (nbh & 7) == 0) {
    const int x = wg & 7, j = wg >> 3, per = nbh >> 3;
    kt_ = j / per;
    bhc_ = (j - kt_ * per) * 8 + x;
  } else {
    bhc_ = VARLEN ? wg % nbh : wg / a.n_tiles;
    kt_ = VARLEN ? wg / nbh : wg - bhc_ * a.n_tiles;
  }
  const int bhc = bhc_;       // (batch, K/V head, chunk), or (sequence, query head)
  const int kt = kt_;         // key tile
  // (batch or sequence, K/V head) and the query head's index in its group.
  int N, bh, chunk;
  size_t base, qbase, lbase, pbase;   // K/V rows, query rows, L/D rows, float32 dK/dV partial rows
  if constexpr (VARLEN) {
    // Rows cu[seq] .. cu[seq+1]-1 of every head (T = a.N rows per head);
    // clamped to the packed tensor and to max_seqlen, so that malformed
    // lengths stay inside the buffers.
    const int T = a.N;
    const int seq = bhc / a.H, h = bhc - seq * a.H;
    int s0 = __builtin_amdgcn_readfirstlane(a.cu_seqlens[seq]);
    int s1 = __builtin_amdgcn_readfirstlane(a.cu_seqlens[seq + 1]);
    s0 = min(max(s0, 0), T);
    s1 = min(max(s1, s0), T);
    N = min(s1 - s0, a.max_seqlen);
    if (kt * kBC >= N) return;   // uniform: the key tile lies past the sequence
    bh = h / a.group;
    chunk = h - bh * a.group;
    base = ((size_t)bh * T + s0) * D;
    qbase = ((size_t)h * T + s0) * D;
    lbase = (size_t)h * T + s0;
    pbase = (((size_t)bh * a.group + chunk) * T + s0) * D;
  } else {
    N = a.N;
    // bhc is the query head (b H + h); its K/V head is bhc / group.
    bh = a.group == 1 ? bhc : bhc / a.group;
    chunk = bhc - bh * a.group;
    const int qh0 = bhc;
    base = (size_t)bh * (size_t)N * D;
    qbase = (size_t)qh0 * (size_t)N * D;
    lbase = (size_t)qh0 * N;
    pbase = ((size_t)bh * a.group + chunk) * (size_t)N * D;
  }
  const unsigned head_bytes = (unsigned)N * C::RB;
  // Query-side buffers start at the group's first head; a visit to head g of
  // the group shifts its offsets by g heads and ends its buffer at head g's
  // last row, so rows past N still read as zero.
  const i32x4 rq = dma_rsrc((const __bf16*)a.q + qbase, head_bytes);
  const i32x4 rk = dma_rsrc((const __bf16*)a.k + base, head_bytes);
  const i32x4 rg = dma_rsrc((const __bf16*)a.dout + qbase, head_bytes);
  const i32x4 rl = dma_rsrc(a.lse + lbase, (unsigned)N * 4);
  const i32x4 rd = dma_rsrc(a.dvec + lbase, (unsigned)N * 4);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const __bf16*)a.v + base, head_bytes);

  const int k0 = kt * kBC;
  const int kw0 = k0 + wave * kKW;
  // dQ destination, addressed by query row: the float32 accumulator of the head.
  const int n_qt = (N + kBR - 1) / kBR;
  const int qt_begin = CAUSAL ? k0 / kBR : 0;
  const int nt = n_qt - qt_begin;   // query tiles visited per query head (>= 1)
  const int nvis = nt;              // visits: query tile n_qt - 1 - i at visit i
  const __amdgpu_buffer_rsrc_t rdq = make_rsrc(a.dq_acc + qbase, (unsigned)N * D * 4);
  const unsigned kt_a = (unsigned)(uintptr_t)LDS(unsigned char, kt_s);
  const unsigned rg_a = (unsigned)(uintptr_t)LDS(unsigned char, rg_s);

  // ---- HBM -> LDS copies (rows past N, and tiles past the end, read as zero).
  auto copy_rows = [&](const i32x4& r, unsigned dst, int row0, int t, bool live) INL {
    const int row = t * C::RPL + lane / C::CPR;
    const int p = lane % C::CPR;
    const unsigned g = live ? (unsigned)(row0 + row) * C::RB + 16 * (p ^ swz<D>(row)) : 0x80000000u;
    dma_load16(r, dst + t * 1024, g);
  };
  // Every wave issues R_LOADS copies per tile: its share of Q and dO, and one
  // copy of L (even waves) or D (odd waves) of the tile's 32 rows; lanes 8..63
  // of that copy read past the row range and write zeros behind it. Two
  // waves copy the same L or D bytes to the same place.
  auto issue_qtile = [&](int i) INL {
    const int qt = n_qt - 1 - i;
    const bool live = i < nvis;
    const unsigned so = rg_a + (i % kStages) * C::STAGE;
#pragma unroll
    for (int u = 0; u < C::QT_LOADS; ++u) {
      const int t = wave * C::QT_LOADS + u;
      copy_rows(rq, so, qt * kBR, t, live);
      copy_rows(rg, so + C::QT, qt * kBR, t, live);
    }
    const unsigned lo = (unsigned)(qt * kBR) * 4 + 16 * lane;
    const unsigned off = live && lane < 8 ? lo : 0x80000000u;
    if (wave & 1)
      dma_load16(rd, so + 2 * C::QT + C::LD, off);
    else
      dma_load16(rl, so + 2 * C::QT, off);
  };


  // K tile (whole workgroup), V operands, then the first two query tiles.
#pragma unroll
  for (int u = 0; u < C::K_LOADS; ++u) copy_rows(rk, kt_a, k0, wave * C::K_LOADS + u, true);
  // V rows of the wave's keys as the B operand of dP = dO V^T (lanes = keys).
  bf16x8 vf[2][C::KSTEPS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const unsigned off = (unsigned)(kw0 + kb * 32 + l32) * C::RB + kk * 32 + hh * 16;
      vf[kb][kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  issue_qtile(0);
  issue_qtile(1);

  // ---- per-lane LDS addresses (byte offsets; chunk bits XORed per step).
  // Rows of a 32-row block read with lanes = one row each (Q, dO: permuted).
  const int prow = acc_row_to_key(l32);
  const int fq_ = swz<D>(prow);
  const unsigned a_lane = (unsigned)prow * C::RB + 16 * ((hh ^ fq_) & 1) + 32 * (fq_ >> 1);
  const int fk = swz<D>(l32);
  const unsigned k_lane = (unsigned)(wave * kKW + l32) * C::RB + 16 * ((hh ^ fk) & 1) + 32 * (fk >> 1);
  // Transposed reads: source lane j = 4s + q of 16-lane group g points at row
  // R0 + s (R0 = 16 * step + 8 * hh + 4 * half), column db*32 + 16*(g%2) + 4q.
  unsigned t_lane[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int b0 = (2 * hh + half) & 3;
    const int hi = D == 128 ? ts : (ts >> 1);
    t_lane[half] = (unsigned)(8 * hh + 4 * half + ts) * C::RB + 64 * hi +
                   16 * ((2 * (g16 & 1) + (tq >> 1)) ^ b0) + 8 * (tq & 1);
  }
  // dS^T tile rows are 64 bytes (32 queries); chunk c of row r sits at c ^ ((r >> 2) & 3).
  unsigned s_lane[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
    s_lane[half] = (unsigned)(8 * hh + 4 * half + ts) * 64 + 16 * ((2 * (g16 & 1) + (tq >> 1)) ^ ((2 * hh + half) & 3)) +
                   8 * (tq & 1);
  const unsigned w_lane = (unsigned)(wave * kKW + l32) * 64;   // dS^T write row base
  const int wsw = (l32 >> 2) & 3;
  // dQ slice of this wave: column block db_q over all 256 keys (NQ steps of
  // 16). For d = 64 waves 0 and 1 form the two column blocks and waves 2
  // and 3 form none (their dQ atomics are no-ops): every dQ element then
  // gets one add per key tile; splitting the keys over two waves per block
  // instead doubles the atomic traffic, which bounds the d = 64 kernel.
  const int db_q = D == 128 ? wave : (wave & 1);
  constexpr int kc_q0 = 0;
  const bool dq_wave = D == 128 || wave < 2;

  f32x16 dk[2][C::DBLK], dv[2][C::DBLK];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
      dk[kb][db] = f32x16{};
      dv[kb][db] = f32x16{};
    }
  const float c = a.c;

  // dQ operands (dS^T and K^T, transposed reads) of product m of the slice.
  auto rd_dq = [&](const unsigned char* sb, int m) INL {
    const int kc = kc_q0 + m;
    Tr4 t;
    t.v[0] = tr_read(sb + s_lane[0] + kc * 16 * 64);
    t.v[1] = tr_read(sb + s_lane[1] + kc * 16 * 64);
    t.v[2] = tr_read(kt_s + (t_lane[0] ^ (64u * db_q)) + kc * 16 * C::RB);
    t.v[3] = tr_read(kt_s + (t_lane[1] ^ (64u * db_q)) + kc * 16 * C::RB);
    return t;
  };
  // dQ atomics of the slice, rows of the query tile of visit `visit`, at the
  // rows' own offsets in rdq. A tile that does not exist (or rows past N)
  // gets offsets past the buffer: the operations are no-ops, so the number
  // of memory operations per tile is the same everywhere.
  auto dq_off = [&](int visit, bool live, int r) INL -> unsigned {
    const int q = (n_qt - 1 - visit) * kBR + 8 * (r >> 2) + 4 * hh + (r & 3);
    return live && q < N ? ((unsigned)q * D + db_q * 32 + l32) * 4 : 0x80000000u;
  };
  auto dq_atomic = [&](const f32x16& acc, int visit, bool live, int r) INL {
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r], rdq, dq_off(visit, live, r), 0, 0);
  };
  constexpr int NDQ = 16;   // dQ memory operations per visit
  auto dq_atomics = [&](const f32x16& acc, int visit, bool live) INL {
#pragma unroll
    for (int r = 0; r < NDQ; ++r) dq_atomic(acc, visit, live, r);
  };

  // ---- fixed-order dQ (DET). Each wave adds to elements no other wave of
  // the workgroup touches (its column block; for d = 64 waves 2 and 3 add
  // nothing and keep their counters in step), so each has a counter (slot)
  // of its own per query tile and waits only on the same wave of lower key
  // tiles: key tile kt's add to a query tile is the kt-th one there.
  const int dq_turn = kt;
  // A device-coherent read of the counter of the tile of `visit` (sc1: the
  // same cache policy as a device-scope atomic load), addressed by scalar
  // registers only, so it holds no vector register but its result.
  const __amdgpu_buffer_rsrc_t rcnt = make_rsrc(a.dq_cnt + (size_t)bhc * n_qt * kBwdSlots, (unsigned)n_qt * kBwdSlots * 4);
  auto dq_peek = [&](int visit) INL -> int {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rcnt, 0, ((n_qt - 1 - visit) * kBwdSlots + wave) * 4, 16);
  };
  // Wait until the earlier contributions to the tile of `visit` are added:
  // the counter is read with device-coherent loads, and this wave's adds are
  // issued only after the load that saw it reach dq_turn has returned. The
  // poll is one assembly block (the load, a compare, a short sleep), so the
  // wait adds no loop to the control flow around the pipelined body (a loop
  // there made the register allocator spill). The wave's polls share one
  // budget over the whole kernel: once it is spent the error flag is set
  // and later waits give up after a single poll, so a wave never polls
  // more than kSpinLimit + visits times.
  unsigned poll_budget = kSpinLimit;
  auto dq_acquire = [&](int visit) INL {
    const int soff = ((n_qt - 1 - visit) * kBwdSlots + wave) * 4;
    int seen, tmp;
    asm volatile(
        "1:\n\t"
        "buffer_load_dword %[t], off, %[r], %[o] sc1\n\t"
        "s_waitcnt vmcnt(0)\n\t"
        "v_readfirstlane_b32 %[v], %[t]\n\t"
        "s_cmp_ge_i32 %[v], %[want]\n\t"
        "s_cbranch_scc1 2f\n\t"
        "s_cmp_eq_u32 %[n], 0\n\t"
        "s_cbranch_scc1 2f\n\t"
        "s_sub_u32 %[n], %[n], 1\n\t"
        "s_sleep 1\n\t"
        "s_branch 1b\n"
        "2:"
        : [t] "=&v"(tmp), [v] "=&s"(seen), [n] "+s"(poll_budget)
        : [r] "s"(rcnt), [o] "s"(soff), [want] "s"(dq_turn)
        : "memory", "scc");
    (void)tmp;
    if (seen < dq_turn) __hip_atomic_store(a.dq_err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // The counter of the tile of `visit` as read during that visit (dq_seen);
  // only if it was not yet this key tile's turn does the wave poll.
  int dq_seen = 0;
  auto dq_wait = [&](int visit) INL {
    if (__builtin_amdgcn_readfirstlane(dq_seen) < dq_turn) dq_acquire(visit);
  };
  // Publish this wave's adds to the tile of `visit`: the caller has waited
  // for every memory operation of the wave to complete (vmcnt 0), so the
  // float adds are done at the device-wide point where atomics are
  // performed before the counter moves. The accumulator is only ever
  // touched by atomics until the kernel ends, so no cache needs writing
  // back or invalidating: the order of the adds is all that is published.
  auto dq_release = [&](int visit) INL {
    asm volatile("" ::: "memory");
    if (lane == 0)
      __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, rcnt, 0, ((n_qt - 1 - visit) * kBwdSlots + wave) * 4, 0);
  };

  __builtin_amdgcn_s_waitcnt(wait_vm(C::R_LOADS));   // K tile, V operands, query tile 0
  lds_barrier();

  // Query tiles are visited from the last one down to the diagonal: the
  // workgroups of one (batch, head) then work on the same rows of dQ at the
  // same time, so its atomics meet in L2 instead of spreading over the whole
  // accumulator. Visit i (query tile qt = n_qt - 1 - i) is in ring stage
  // i % 3; its dS^T goes to dS buffer i % 2, which dQ of visit i reads during
  // visit i + 1.
  for (int i = 0; i < nvis; ++i) {
    const int qt = n_qt - 1 - i;
    if (i > 0) {
      if constexpr (DET) {
        // Only the NDQ dQ atomics of visit i-1 may stay in flight: the
        // copies of visits i and i+1, the atomics of visit i-2 (those of
        // visit i-3's tile, published here) and the counter read of visit
        // i-1 have landed. That read decides whether this visit's adds (to
        // visit i-1's tile) may go ahead or must wait.
        __builtin_amdgcn_s_waitcnt(wait_vm(NDQ));
        lds_barrier();
        if (i >= 3) dq_release(i - 3);
        dq_wait(i - 1);
      } else {
        // Memory operations issued after visit i's own copies: (i >= 2) the NDQ
        // dQ operations of visit i-2, then the copies of visit i+1 and the NDQ
        // dQ operations of visit i-1.
        if (i == 1)
          __builtin_amdgcn_s_waitcnt(wait_vm(C::R_LOADS + NDQ));
        else
          __builtin_amdgcn_s_waitcnt(wait_vm(C::R_LOADS + 2 * NDQ));
        lds_barrier();
      }
    }

    const int q0 = qt * kBR;
    const unsigned char* qs = ring(i % kStages);
    const unsigned char* sb_prev = dsb((i + 1) & 1);
    // Waves whose keys all follow the tile's rows run the tile fully masked.
    const bool active = !CAUSAL || kw0 <= q0 + kBR - 1;
    const bool mask = !active || kw0 + kKW > N || (CAUSAL && kw0 + kKW - 1 > q0);
    int lim[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kw0 + kb * 32 + l32;
      lim[kb] = !mask ? -1 : (!active || key >= N) ? kBR : CAUSAL ? key - q0 : -1;
    }

    // ---- d = 64: both key blocks in one pass (the visit is bound by its
    // LDS reads and round trips, not by the matrix cores): phase A forms S
    // and dP of both blocks one d step at a time, so every Q and dO
    // fragment feeds two products; phase B runs the softmax of both blocks
    // beside the dQ products of visit i-1; phase C writes dS^T and forms
    // dV and dK of both blocks, each transposed operand read once for both,
    // with the dQ atomics of visit i-1 spread over its steps.
    if constexpr (D == 64) {
      // L and D of row slot r = query slot_key(r, hh): slots 4 q .. 4 q + 3
      // are 4 consecutive rows, one 16-byte read each.
      const float* Ls = (const float*)(qs + 2 * C::QT);
      const float* Ds = (const float*)(qs + 2 * C::QT + C::LD);
      struct LD4 {
        float l[4], d[4];   // L log2 e and D of 4 row slots
      };
      auto rd_ld4 = [&](int q) INL {
        LD4 v;
        const int o = 16 * (q >> 1) + 8 * hh + 4 * (q & 1);
        const f32x4 l0 = *LDS(const f32x4, Ls + o), d0 = *LDS(const f32x4, Ds + o);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v.l[t] = l0[t] * kLog2e;
          v.d[t] = d0[t];
        }
        return v;
      };
      f32x16 s[2], dp[2];
      bf16x8 pf[2][2], df[2][2];
      auto soft = [&](int kb, int r, float l2, float dd) INL {
        const int ql = slot_key(r, hh);
        float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -l2));
        p = ql >= lim[kb] ? p : 0.f;
        const float ds = p * (dp[kb][r] - dd);
        pf[kb][r >> 3][r & 7] = (__bf16)p;
        df[kb][r >> 3][r & 7] = (__bf16)ds;
      };
      // Phase A.
      bf16x8 fq[2], fg[2], fk0[2], fk1[2];
      auto rd_a = [&](int kk) INL {
        const int b = kk % 2;
        fq[b] = *LDS(bf16x8, qs + (a_lane ^ (32u * kk)));
        fg[b] = *LDS(bf16x8, qs + C::QT + (a_lane ^ (32u * kk)));
        fk0[b] = *LDS(bf16x8, kt_s + (k_lane ^ (32u * kk)));
        fk1[b] = *LDS(bf16x8, kt_s + (k_lane ^ (32u * kk)) + 32 * C::RB);
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
      }
      rd_a(0);
#pragma unroll
      for (int kk = 0; kk < C::KSTEPS; ++kk) {
        const int b = kk % 2;
        if (kk + 1 < C::KSTEPS) rd_a(kk + 1);
        // Copies of visit i+2 go to the stage of visit i-1 (free since the
        // barrier); issued here rather than right after the barrier, where
        // they would queue behind the previous visit's dQ atomics and stall.
        if (kk == C::KSTEPS / 2) issue_qtile(i + 2);
        __builtin_amdgcn_sched_barrier(0);
        s[0] = mma(fq[b], fk0[b], s[0]);
        dp[0] = mma(fg[b], vf[0][kk], dp[0]);
        s[1] = mma(fq[b], fk1[b], s[1]);
        dp[1] = mma(fg[b], vf[1][kk], dp[1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // Phase B: an equal share of the 32 evaluations per dQ product; dQ
      // operands one product ahead, L and D one quarter of the slots ahead.
      // Waves that form no dQ run the evaluations alone.
      constexpr int EPM = 32 / C::NQ;
      static_assert(EPM * C::NQ == 32 && C::NQ % 4 == 0, "evaluation split");
      constexpr int MQ = C::NQ / 4;   // products per quarter of the slots
      f32x16 dq_acc = f32x16{};
      auto phase_b = [&](auto with_dq) INL {
        constexpr bool WQ = decltype(with_dq)::value != 0;
        LD4 ldq[2];
        ldq[0] = rd_ld4(0);
        Tr4 qop[2];
        if constexpr (WQ) qop[0] = rd_dq(sb_prev, 0);
#pragma unroll
        for (int m = 0; m < C::NQ; ++m) {
          if constexpr (WQ) {
            if (m + 1 < C::NQ) qop[(m + 1) % 2] = rd_dq(sb_prev, m + 1);
          }
          if (m % MQ == 0 && m / MQ + 1 < 4) ldq[(m / MQ + 1) % 2] = rd_ld4(m / MQ + 1);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (WQ)
            dq_acc = mma(join(qop[m % 2].v[0], qop[m % 2].v[1]), join(qop[m % 2].v[2], qop[m % 2].v[3]), dq_acc);
#pragma unroll
          for (int t = 0; t < EPM; ++t) {
            const int e = m * EPM + t, r = e >> 1, kb = e & 1;
            soft(kb, r, ldq[(r >> 2) % 2].l[r & 3], ldq[(r >> 2) % 2].d[r & 3]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (dq_wave)
        phase_b(IC<1>{});
      else
        phase_b(IC<0>{});
      // Phase C.
      {
        // dS^T rows (keys) of this wave: 8 queries per 16-byte write.
        unsigned char* sp = dsb(i & 1) + w_lane;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) *LDS(bf16x8, sp + kb * 32 * 64 + 16 * ((2 * k2 + hh) ^ wsw)) = df[kb][k2];
      }
      auto trd = [&](int step) INL {
        const int ks = step / C::DBLK, db = step % C::DBLK;
        const unsigned char* ko = qs + ks * 16 * C::RB;
        Tr4 t;
        t.v[0] = tr_read(ko + C::QT + (t_lane[0] ^ (64u * db)));
        t.v[1] = tr_read(ko + C::QT + (t_lane[1] ^ (64u * db)));
        t.v[2] = tr_read(ko + (t_lane[0] ^ (64u * db)));
        t.v[3] = tr_read(ko + (t_lane[1] ^ (64u * db)));
        return t;
      };
      constexpr int NS = 2 * C::DBLK;   // (ks, db) steps
      auto dvdk = [&](int kb, const Tr4& t, int step) INL {
        const int ks = step / C::DBLK, db = step % C::DBLK;
        dv[kb][db] = mma(pf[kb][ks], join(t.v[0], t.v[1]), dv[kb][db]);
        dk[kb][db] = mma(df[kb][ks], join(t.v[2], t.v[3]), dk[kb][db]);
      };
      Tr4 top[2];
      top[0] = trd(0);
#pragma unroll
      for (int step = 0; step < NS; ++step) {
        const int b = step % 2;
        if (step + 1 < NS) top[(step + 1) % 2] = trd(step + 1);
        __builtin_amdgcn_sched_barrier(0);
        dvdk(0, top[b], step);
        dvdk(1, top[b], step);
        // Fixed order: read the counter of this visit's own tile now (the
        // next visit adds to it); its value is needed only after the next
        // barrier, so the read costs no wait.
        if constexpr (DET) {
          if (step == 0) dq_seen = dq_peek(i);
        }
        // dQ memory operations r in [lo, hi) of the NDQ, split evenly over the steps
        const int lo = step * NDQ / NS, hi = (step + 1) * NDQ / NS;
#pragma unroll
        for (int r = lo; r < hi; ++r) dq_atomic(dq_acc, i - 1, i > 0 && dq_wave, r);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // L and D of the tile's rows (each lane reads those of its row slots).
      const float* Ls = (const float*)(qs + 2 * C::QT);
      const float* Ds = (const float*)(qs + 2 * C::QT + C::LD);
      // Softmax of row slot r of key block kb: P = exp2(S c - L log2 e), dS =
      // P (dP - D). Entry (q0 + ql, key) is kept iff ql >= lim.
      f32x16 s[2], dp[2];
      bf16x8 pf[2][2], df[2][2];
      constexpr int SPK = 16 / C::KSTEPS;   // softmax evaluations per d step (= per dV/dK step)
      static_assert(SPK == 16 / (2 * C::DBLK), "one evaluation count per step");
      // L (times log2 e) and D of the row slots r0 .. r0+SPK-1, read from LDS one
      // step before their use, ahead of that step's operand reads: waiting for
      // them then never waits for the operands of the step after.
      struct LDv {
        float l[SPK], d[SPK];
      };
      auto rd_ld = [&](int r0) INL {
        LDv v;
  #pragma unroll
        for (int t = 0; t < SPK; ++t) {
          const int ql = slot_key(r0 + t, hh);
          v.l[t] = *LDS(const float, Ls + ql);
          v.d[t] = *LDS(const float, Ds + ql);
        }
        return v;
      };
      auto soft = [&](int kb, int r, const LDv& ld) INL {
        const int ql = slot_key(r, hh);
        const float l2 = ld.l[r % SPK] * kLog2e, dd = ld.d[r % SPK];
        float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -l2));
        p = ql >= lim[kb] ? p : 0.f;
        const float ds = p * (dp[kb][r] - dd);
        pf[kb][r >> 3][r & 7] = (__bf16)p;
        df[kb][r >> 3][r & 7] = (__bf16)ds;
      };

      // ---- Phase 1: S and dP of tile i for key block 0, then for key block 1
      // beside the softmax of block 0 (two evaluations per d step); operands
      // read one step ahead.
      bf16x8 fq[2], fg[2], fk[2];
      LDv ldv[2];
      auto rd_sdp = [&](int kb, int kk) INL {
        const int b = kk % 2;
        fq[b] = *LDS(bf16x8, qs + (a_lane ^ (32u * kk)));
        fg[b] = *LDS(bf16x8, qs + C::QT + (a_lane ^ (32u * kk)));
        fk[b] = *LDS(bf16x8, kt_s + (k_lane ^ (32u * kk)) + kb * 32 * C::RB);
      };
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // Copies of visit i+2 go to the stage of visit i-1 (free since the
        // barrier). Issued here rather than right after the barrier, where
        // they would queue behind the previous visit's dQ atomics and stall.
        if (kb == 1) issue_qtile(i + 2);
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
        if (kb == 1) ldv[0] = rd_ld(0);
        rd_sdp(kb, 0);
  #pragma unroll
        for (int kk = 0; kk < C::KSTEPS; ++kk) {
          const int b = kk % 2;
          if (kk + 1 < C::KSTEPS) {
            if (kb == 1) ldv[(kk + 1) % 2] = rd_ld((kk + 1) * SPK);
            rd_sdp(kb, kk + 1);
          }
          __builtin_amdgcn_sched_barrier(0);
          s[kb] = mma(fq[b], fk[b], s[kb]);
          dp[kb] = mma(fg[b], vf[kb][kk], dp[kb]);
          if (kb == 1) {
  #pragma unroll
            for (int t = 0; t < SPK; ++t) soft(0, kk * SPK + t, ldv[b]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- Phase 2: dV += P^T dO and dK += dS^T Q of key block 0 beside the
      // softmax of key block 1; phase 3: the same products of key block 1 with
      // dQ of visit i-1 (its dS^T is complete in LDS) interleaved. The B operands
      // of dV and dK are read transposed from the ring one (ks, db) step ahead
      // (once per key block); the dQ operands one product ahead.
      auto trd = [&](int step) INL {
        const int ks = step / C::DBLK, db = step % C::DBLK;
        const unsigned char* ko = qs + ks * 16 * C::RB;
        Tr4 t;
        t.v[0] = tr_read(ko + C::QT + (t_lane[0] ^ (64u * db)));
        t.v[1] = tr_read(ko + C::QT + (t_lane[1] ^ (64u * db)));
        t.v[2] = tr_read(ko + (t_lane[0] ^ (64u * db)));
        t.v[3] = tr_read(ko + (t_lane[1] ^ (64u * db)));
        return t;
      };
      constexpr int NS = 2 * C::DBLK;   // (ks, db) steps per key block
      auto dvdk = [&](int kb, const Tr4& t, int step) INL {
        const int ks = step / C::DBLK, db = step % C::DBLK;
        dv[kb][db] = mma(pf[kb][ks], join(t.v[0], t.v[1]), dv[kb][db]);
        dk[kb][db] = mma(df[kb][ks], join(t.v[2], t.v[3]), dk[kb][db]);
      };
      Tr4 top[2];
      ldv[0] = rd_ld(0);
      top[0] = trd(0);
      constexpr int SPS = SPK;          // softmax evaluations per step
  #pragma unroll
      for (int step = 0; step < NS; ++step) {
        const int b = step % 2;
        if (step + 1 < NS) {
          ldv[(step + 1) % 2] = rd_ld((step + 1) * SPS);
          top[(step + 1) % 2] = trd(step + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        dvdk(0, top[b], step);
  #pragma unroll
        for (int t = 0; t < SPS; ++t) soft(1, step * SPS + t, ldv[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        // dS^T rows (keys) of this wave: 8 queries per 16-byte write.
        unsigned char* sp = dsb(i & 1) + w_lane;
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) *LDS(bf16x8, sp + kb * 32 * 64 + 16 * ((2 * k2 + hh) ^ wsw)) = df[kb][k2];
      }
      top[0] = trd(0);
      Tr4 qop[2];
      qop[0] = rd_dq(sb_prev, 0);
      f32x16 dq_acc = f32x16{};
      // dQ products in the first quarter of the steps, its atomics spread over
      // the rest (one burst of 16 would stall on vector-memory issue).
      constexpr int QS = NS / 4;                 // steps that carry dQ products
      constexpr int QPS = C::NQ / QS;            // dQ products per such step
  #pragma unroll
      for (int step = 0; step < NS; ++step) {
        const int b = step % 2;
        if (step + 1 < NS) top[(step + 1) % 2] = trd(step + 1);
        __builtin_amdgcn_sched_barrier(0);
        dvdk(1, top[b], step);
        if (step < QS) {
  #pragma unroll
          for (int t = 0; t < QPS; ++t) {
            const int m = step * QPS + t;
            if (m + 1 < C::NQ) qop[(m + 1) % 2] = rd_dq(sb_prev, m + 1);
            dq_acc = mma(join(qop[m % 2].v[0], qop[m % 2].v[1]), join(qop[m % 2].v[2], qop[m % 2].v[3]), dq_acc);
          }
        } else {
          // Fixed order: read the counter of this visit's own tile now (the
          // next visit adds to it); its value is needed only after the next
          // barrier, so the read costs no wait.
          if constexpr (DET) {
            if (step == QS) dq_seen = dq_peek(i);
          }
          // memory operations r in [lo, hi) of the NDQ, split evenly over steps QS .. NS-1
          constexpr int NA = NS - QS;
          const int lo = (step - QS) * NDQ / NA, hi = (step - QS + 1) * NDQ / NA;
  #pragma unroll
          for (int r = lo; r < hi; ++r) dq_atomic(dq_acc, i - 1, i > 0, r);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

    }
  }

  // dQ of the last visited tile.
  if constexpr (DET) {
    __builtin_amdgcn_s_waitcnt(wait_vm(NDQ));
    lds_barrier();
    if (nvis >= 3) dq_release(nvis - 3);
    dq_wait(nvis - 1);
  } else {
    lds_barrier();
  }
  {
    const unsigned char* sb = dsb((nvis - 1) & 1);
    Tr4 qop[3];
    f32x16 dq_acc = f32x16{};
    if (dq_wave) {
      qop[0] = rd_dq(sb, 0);
      qop[1] = rd_dq(sb, 1);
#pragma unroll
      for (int m = 0; m < C::NQ; ++m) {
        if (m + 2 < C::NQ) qop[(m + 2) % 3] = rd_dq(sb, m + 2);
        __builtin_amdgcn_sched_barrier(0);
        dq_acc = mma(join(qop[m % 3].v[0], qop[m % 3].v[1]), join(qop[m % 3].v[2], qop[m % 3].v[3]), dq_acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    dq_atomics(dq_acc, nvis - 1, dq_wave);
    if constexpr (DET) {
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
      if (nvis >= 2) dq_release(nvis - 2);
      dq_release(nvis - 1);
    }
  }

  // Epilogue: dK = scale * acc, dV = acc (lanes = d, rows = keys); rows past N dropped.
  if (a.dkv_part != nullptr) {
    // float32 dK and dV of this chunk: [batch, K/V head][chunk][N][d] each
    // (VARLEN: [K/V head][chunk][T][d], this sequence's rows).
    const size_t pb = pbase;
    const size_t half = (size_t)a.H * (size_t)a.N * D * (size_t)(a.B);
    const __amdgpu_buffer_rsrc_t rpk = make_rsrc(a.dkv_part + pb, (unsigned)N * D * 4);
    const __amdgpu_buffer_rsrc_t rpv = make_rsrc(a.dkv_part + half + pb, (unsigned)N * D * 4);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kw0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          const unsigned off = ((unsigned)key * D + db * 32 + l32) * 4;
          const float kx = dk[kb][db][r] * a.scale, vx = dv[kb][db][r];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, kx), rpk, off, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, vx), rpv, off, 0, 0);
        }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    return;
  }
  const __amdgpu_buffer_rsrc_t rdk = make_rsrc((__bf16*)a.dk + base, head_bytes);
  const __amdgpu_buffer_rsrc_t rdv = make_rsrc((__bf16*)a.dv + base, head_bytes);
  const float scale = a.scale;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kw0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const unsigned off = (unsigned)key * C::RB + 2 * (db * 32 + l32);
        const __bf16 kv = (__bf16)(dk[kb][db][r] * scale);
        const __bf16 vv = (__bf16)dv[kb][db][r];
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, kv), rdk, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, vv), rdv, off, 0, 0);
      }
  // Copies of tiles past the end (zeros into free ring stages) may still be
  // in flight: let them land before the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
#endif
}

template <int D, bool CAUSAL, bool DET>
void launch_main(const BwdArgs& a, long long grid, hipStream_t s) {
  if (a.cu_seqlens != nullptr)   // packed variable-length batch
    hipLaunchKernelGGL((bwd_bf16_kernel<D, CAUSAL, false, true>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_bf16_kernel<D, CAUSAL, DET, false>), dim3(grid), dim3(kThreads), 0, s, a);
}

}  // namespace

hipError_t launch_bwd_bf16_main(int d, int causal, BwdArgs a, int B, int H, hipStream_t s) {
  // One workgroup per (batch, query head, key tile), or, for a packed
  // variable-length batch, per (sequence, query head, key tile of the
  // longest sequence).
  a.n_tiles = ((a.cu_seqlens != nullptr ? a.max_seqlen : a.N) + kBC - 1) / kBC;
  const long long grid = a.cu_seqlens != nullptr ? (long long)a.n_seq * H * a.n_tiles
                                                 : (long long)B * H * a.n_tiles;
  a.remap = grid % 8 == 0 ? 1 : 0;
  const bool det = a.dq_cnt != nullptr;
  if (d == 64) {
    if (causal) det ? launch_main<64, true, true>(a, grid, s) : launch_main<64, true, false>(a, grid, s);
    else det ? launch_main<64, false, true>(a, grid, s) : launch_main<64, false, false>(a, grid, s);
  } else {
    if (causal) det ? launch_main<128, true, true>(a, grid, s) : launch_main<128, true, false>(a, grid, s);
    else det ? launch_main<128, false, true>(a, grid, s) : launch_main<128, false, false>(a, grid, s);
  }
  return hipGetLastError();
}

}  // namespace fa
