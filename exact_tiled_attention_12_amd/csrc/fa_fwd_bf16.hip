// Fused exact-attention forward, bf16, for gfx950 (MI355X).
//
// What it computes ("FlashAttention v1～v4 完整进化史", v1 pseudocode and v2
// part 1; "6.1 FlashAttention V1详解", section 5.1): per query row the running
// maximum m, the exponent sum l and an unnormalised output accumulator are
// carried across the key/value tiles, and O = acc / l, L = m + log l are
// written once. Scores and probabilities stay in registers.
//
// Schedule:
//   * one workgroup = 8 waves = 256 query rows of one (batch, head); each
//     wave owns 32 rows; the grid issues the heaviest causal tiles first and
//     groups the tiles of a (batch, head) on one XCD. For d = 64 and a small
//     grid, workgroups of 4 waves (128 rows) whose ring takes half the LDS,
//     so that two share a CU and the work spreads over more of them;
//   * K and V tiles of 64 keys move from HBM straight into a 5-stage LDS ring
//     (buffer loads with an LDS destination; rows past N read as zero), with
//     one workgroup barrier per tile; a tile is resident two steps before
//     its first read so that each step can fetch the first operands of the
//     next one;
//   * S^T = K Q^T and O^T = V^T P^T on the 32x32x16 bf16 MFMA: K rows are read
//     in a permuted order so every lane owns one query and holds its
//     exponentiated scores in exactly the operand layout of the second
//     product; V stays row-major in LDS and is read transposed with
//     ds_read_b64_tr_b16;
//   * the work is a software pipeline over 32-key blocks: step u forms the
//     exponentials of block u while the matrix cores run S of block u+1 and
//     the product of block u-1 with V. None of the step's 16 products depends
//     on its vector work, so the two are interleaved instruction by
//     instruction (scheduling groups) and the matrix cores need not wait for
//     the softmax;
//   * lazy re-basing ("FlashAttention v1～v4 完整进化史", v4 part 3):
//     exponentials are taken against a reference maximum m_ref that is moved
//     only when needed. A step first exponentiates against the current
//     m_ref; if the block sum of some lane is above 2^8 (or not finite, as in
//     the first block, where m_ref = -inf), the wave takes the row maxima,
//     re-bases every row to max(m_ref, row max), rescales l and the
//     accumulator, and redoes the exponentials. Otherwise every exponential
//     is below 2^8 and no maximum is formed at all. O / l and m_ref + log l
//     are exact whatever m_ref is, so this only reorders the arithmetic;
//   * LDS rows are XOR-swizzled per 16-byte chunk so the K reads (16 rows, one
//     chunk) and the transposed V reads (4 rows x 4 chunks) are free of bank
//     conflicts.
#include <cfloat>
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kBC = 64;            // keys per tile
constexpr int kStages = 5;
// A lane's exponent sum over one 16-score half block above this (2^8) or not
// finite triggers a re-base; below it every exponential is below 2^8.
constexpr float kPartMax = 256.f;

template <int N>
using IC = std::integral_constant<int, N>;

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS(T, p) ((__attribute__((address_space(3))) T*)(p))
// The kernel body is built from lambdas; each must be inlined (a call would
// move the accumulators through scratch memory).
#define INL __attribute__((always_inline)) __device__

// W waves per workgroup (32 query rows each). With 8 waves one workgroup
// fills a CU (two waves per SIMD); with 4 (d = 64 only) two workgroups share
// a CU, each ring taking half of its LDS.
template <int D, int W>
struct Cfg {
  static constexpr int WAVES = W;
  static constexpr int THREADS = 64 * W;
  static constexpr int BR = 32 * W;                 // query rows per workgroup
  static constexpr int WG_PER_CU = W == 4 ? 2 : 1;
  static constexpr int RB = D * 2;                  // bytes per row
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row
  static constexpr int TILE = kBC * RB;             // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int LDS_BYTES = kStages * STAGE;
  static constexpr int LPW = TILE / 1024 / W;       // 1 KiB wave-loads per wave per tensor
  static constexpr int RPL = 1024 / RB;             // rows per wave-load
  static constexpr int LOADS = 2 * LPW;             // loads per wave per tile
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static_assert(W == 4 || W == 8, "waves per workgroup");
  static_assert((LPW == 1 || LPW == 2) && LPW * W * 1024 == TILE, "tile split");
  static_assert(WG_PER_CU * LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(2 * LOADS <= 15, "vmcnt immediates below assume waits for at most 15 loads");
};

// Physical chunk of logical chunk c in LDS row r. K: the 16 rows read together
// by one 16-lane group land on 16 distinct bank groups. V: 4 consecutive rows
// x 4 consecutive chunks (one ds_read_b64_tr_b16 group) do.
template <int D>
__device__ __forceinline__ int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_swz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Transposed 64-bit LDS read (see the V fragment layout below).
__device__ __forceinline__ u32x2 tr_read(const unsigned char* lds_byte_ptr) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS(i16x4, lds_byte_ptr)));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Workgroup barrier for the LDS ring, ordering LDS only: each wave first
// waits (vmcnt) for its own loads of the tile to land; loads still in flight
// to other stages stay in flight.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// VARLEN: packed variable-length batch; a workgroup of a tile past its
// sequence's end exits at once.
// SKIP (causal only): a wave stops computing once every block a step
// touches lies above its rows, and from then on only issues its share of the
// tile loads and keeps the barriers. It pays on short causal sequences,
// where the diagonal tiles are a larger share of the work; on long ones the
// branch's registers cost more than it saves.
template <int D, int W, bool CAUSAL, bool VARLEN, bool SKIP>
__global__ __launch_bounds__(64 * W, W == 4 ? 2 : 1) void fwd_bf16_kernel(FwdArgs a) {
  // The body is compiled in the device pass only: the host pass needs just the
  // launch stub, and its front end drops the stub of a kernel whose lambdas
  // capture buffer resources.
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg<D, W>;
  constexpr int kBR = C::BR;
  // One variable per ring stage: with the stage known at compile time the
  // compiler can tell a tile being read from the tiles being loaded, and needs
  // no wait on the in-flight loads before the reads.
  __shared__ __attribute__((aligned(1024))) unsigned char st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st4[C::STAGE];
  auto sp = [&](auto stag) -> unsigned char* {
    constexpr int S = decltype(stag)::value;
    if constexpr (S == 0) return st0;
    else if constexpr (S == 1) return st1;
    else if constexpr (S == 2) return st2;
    else if constexpr (S == 3) return st3;
    else return st4;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  // Work items are (batch or sequence, head, query tile). With more items
  // than CUs and the (batch, head) pairs a multiple of 8, the launch is
  // persistent: one workgroup per CU, and the workgroups of XCD x (ids go to
  // the XCDs round-robin) take the items 8 m + x of that XCD, round by round
  // in snake order (round r: m = r S + j, or r S + S - 1 - j when r is odd,
  // for the XCD's S workgroups j), so that with items in decreasing order of
  // work every workgroup gets about the same total; a workgroup then starts
  // its next item without a new launch. Otherwise one item per workgroup.
  for (int round = 0;; ++round) {
  int wg, nsh;   // item, (batch or sequence, head) pairs
  if (!VARLEN && a.persist) {
    const int S = (int)gridDim.x >> 3, x = (int)blockIdx.x & 7, j = (int)blockIdx.x >> 3;
    const int m = round * S + ((round & 1) ? S - 1 - j : j);
    wg = 8 * m + x;
    if (wg >= a.n_items) break;
    nsh = a.n_items / a.n_qtiles;
  } else {
    if (round > 0) break;
    wg = blockIdx.x;
    nsh = gridDim.x / a.n_qtiles;
  }
  int bh, t;
  // Causal or packed variable-length, with the (batch or sequence, head)
  // pairs a multiple of 8: each pair stays on one XCD and every XCD runs its
  // pairs' tiles tile-major, the heaviest tiles (the last ones, of the
  // longest sequences) first. Otherwise the tiles of one pair are grouped on
  // one XCD and run in order (causal: heaviest first); with equal tiles that
  // keeps a head's K/V in L2.
  if ((CAUSAL || VARLEN) && a.remap && (nsh & 7) == 0) {
    const int x = wg & 7, j = wg >> 3;           // XCD, position within it
    const int per = nsh >> 3;
    t = j / per;
    bh = (j - t * per) * 8 + x;
  } else if (!VARLEN && a.persist) {
    // equal tiles: the XCD's heads one after the other
    const int x = wg & 7, m = wg >> 3;
    const int hx = m / a.n_qtiles;
    bh = hx * 8 + x;
    t = m - hx * a.n_qtiles;
  } else {
    if (a.remap) wg = xcd_remap(wg, gridDim.x);
    bh = wg / a.n_qtiles;   // (batch, head), or (sequence, head) for VARLEN
    t = wg - bh * a.n_qtiles;
  }
  const int qt = CAUSAL ? (a.n_qtiles - 1 - t) : t;
  int N = a.N;
  size_t base, kv_base, lse_base;
  if constexpr (VARLEN) {
    // Rows cu[seq] .. cu[seq+1]-1 of every head; clamped to the packed
    // tensor and to the longest-sequence bound, so that malformed lengths
    // stay inside the buffers.
    const int seq = bh / a.H, h = bh - seq * a.H;
    int s0 = __builtin_amdgcn_readfirstlane(a.cu_seqlens[seq]);
    int s1 = __builtin_amdgcn_readfirstlane(a.cu_seqlens[seq + 1]);
    s0 = min(max(s0, 0), a.N);
    s1 = min(max(s1, s0), a.N);
    N = min(s1 - s0, a.n_qtiles * kBR);
    if (qt * kBR >= N) continue;   // uniform: the tile lies past the sequence
    const int kvh = h / a.group;
    base = ((size_t)h * a.N + s0) * D;
    kv_base = ((size_t)kvh * a.N + s0) * D;
    lse_base = (size_t)h * a.N + s0;
  } else {
    base = (size_t)bh * (size_t)N * D;
    // K/V head of this query head: groups of `group` consecutive query heads
    // share one (grouped-query attention; group = 1 is one K/V head per head).
    const int kvh = a.group == 1 ? bh : (bh / a.H) * (a.H / a.group) + (bh % a.H) / a.group;
    kv_base = (size_t)kvh * (size_t)N * D;
    lse_base = (size_t)bh * N;
  }
  const unsigned head_bytes = (unsigned)N * C::RB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const __bf16*)a.q + base, head_bytes);
  const i32x4 rk = dma_rsrc((const __bf16*)a.k + kv_base, head_bytes);
  const i32x4 rv = dma_rsrc((const __bf16*)a.v + kv_base, head_bytes);

  const int q0 = qt * kBR;
  const int wrow0 = q0 + wave * 32;
  const int qrow = wrow0 + l32;

  const int n_kv = (N + kBC - 1) / kBC;
  const int kv_end = CAUSAL ? min(n_kv, (min(q0 + kBR, N) - 1) / kBC + 1) : n_kv;
  const int U = 2 * kv_end;   // 32-key blocks

  // --- tile loads: HBM -> LDS, no registers. Wave-load t covers rows
  // [t*RPL, t*RPL+RPL) of the tile; lane l fills physical chunk l % CPR of
  // row t*RPL + l / CPR with the logical chunk that the swizzle maps there.
  // Each wave issues 2*LPW loads (K and V, part i) per tile. A tile index at
  // or past kv_end gets an offset past the buffer end: the load moves no data
  // and writes zeros to a stage nobody reads, which keeps the number of loads
  // in flight the same for every tile.
  auto issue_load = [&](int j, auto stag, int i, bool is_v) INL {
    const int tl = wave * C::LPW + i;
    const int row = tl * C::RPL + lane / C::CPR;
    const int p = lane % C::CPR;
    const unsigned grow = j < kv_end ? (unsigned)(j * kBC + row) * C::RB : 0x80000000u;
    const unsigned d = (unsigned)(uintptr_t)LDS(unsigned char, sp(stag)) + tl * 1024 + (is_v ? C::TILE : 0);
    if (is_v)
      dma_load16(rv, d, grow + 16 * (p ^ v_swz<D>(row)));
    else
      dma_load16(rk, d, grow + 16 * (p ^ k_swz<D>(row)));
  };
  auto issue_tile = [&](int j, auto stag) INL {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      issue_load(j, stag, i, false);
      issue_load(j, stag, i, true);
    }
  };

  // --- Q rows of this wave as the B operand of S^T = K Q^T (rows past N read 0).
  bf16x8 qf[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
    const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        rq, (unsigned)qrow * C::RB + kk * 32 + hh * 16, 0, 0));
    qf[kk] = __builtin_bit_cast(bf16x8, w);
  }
  // Q must be complete before tile loads are queued behind it (the loop's
  // waits are then only for tiles).
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // --- per-lane LDS read addresses (byte offsets inside a stage).
  // K fragment (key block kb, d step kk) of lane (l32, hh): row kb*32 +
  // acc_row_to_key(l32), logical chunk 2*kk + hh. Row bases are multiples of
  // 256 (D=128) or 128 (D=64) so chunk bits can be XORed into the address.
  const int prow = acc_row_to_key(l32);
  const unsigned k_lane = (unsigned)prow * C::RB + 16 * (hh ^ (k_swz<D>(prow) & 1)) + 32 * (k_swz<D>(prow) >> 1);
  // V fragment: source lane j = 4s + q of 16-lane group g points at row
  // R0 + s, columns db*32 + 16*(g%2) + 4q (R0 is a multiple of 4). The d
  // block only flips address bits 6-7 (64 * (db ^ swizzle)), so one lane
  // address serves every block through an XOR.
  const int g16 = lane >> 4, j16 = lane & 15;
  const int vs = j16 >> 2, vq = j16 & 3;
  const unsigned v_lane = (unsigned)(vs + 8 * hh) * C::RB + 16 * ((2 * (g16 & 1) + (vq >> 1)) ^ v_swz<D>(vs)) +
                          8 * (vq & 1);

  const float c = a.c;
  float m_ref = -INFINITY;   // reference maximum (scaled log2 units) of this lane's row
  float l = 0.f;             // exponent sum over this lane half's keys, against m_ref
  f32x16 oacc[C::DBLK];
#pragma unroll
  for (int i = 0; i < C::DBLK; ++i) oacc[i] = f32x16{};

  // K fragments of 32-key block `kblk` of the tile in stage `kst`.
  auto read_k = [&](auto kst, auto kblk, bf16x8 (&kf)[C::KSTEPS]) INL {
    const unsigned char* kt = sp(kst) + decltype(kblk)::value * 32 * C::RB;
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) kf[kk] = *LDS(bf16x8, kt + (k_lane ^ (32u * kk)));
  };
  // Scores of block u that are past N or (causal) above the diagonal -> -inf.
  // Needed on ragged and diagonal blocks only; blocks entirely past the last
  // row of the wave come out fully masked and add nothing.
  auto masked = [&](int u) INL { return u * 32 + 32 > N || (CAUSAL && u * 32 + 31 > wrow0); };
  auto apply_mask = [&](int u, f32x16& s) INL {
    const int key0 = u * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + slot_key(r, hh);
      const bool ok = key < N && (!CAUSAL || key <= qrow);
      s[r] = ok ? s[r] : -INFINITY;
    }
  };

  // Exponentials of one block against m_sub, packed to bf16 as the operand of
  // the product with V; returns this lane's sum of the (unrounded) values.
  // c > 0 (the launcher clamps it), so masked scores give exactly 0.
  auto exps = [&](const f32x16& s, float m_sub, bf16x8 (&p)[2]) INL -> float {
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(__builtin_fmaf(s[r], c, -m_sub));
      part[r & 3] += e;
      p[r >> 3][r & 7] = (__bf16)e;
    }
    return (part[0] + part[1]) + (part[2] + part[3]);
  };

  // Order of the 2*KSTEPS products of a step: S (K fragment i) and O (V
  // fragment i) alternate, except that the last two S products come before
  // the last two O products, so S of the next block is complete two products
  // before the next step reads it.
  constexpr int NM = 2 * C::KSTEPS;
  auto pos_is_s = [](int p) constexpr { return p < NM - 4 ? p % 2 == 0 : (p == NM - 4 || p == NM - 3); };
  auto pos_idx = [](int p) constexpr {
    return p < NM - 4 ? p / 2 : (p == NM - 4 ? NM / 2 - 2 : p == NM - 3 ? NM / 2 - 1 : p == NM - 2 ? NM / 2 - 2 : NM / 2 - 1);
  };
  constexpr int AHEAD = 3;   // operands are read this many products ahead
  struct Ops {
    bf16x8 kf[C::KSTEPS];
    bf16x8 vf[2 * C::DBLK];
  };
  // Operand of the product at position p, from the K tile kt / V tile vt.
  auto fetch = [&](int p, Ops& o, const unsigned char* kt, const unsigned char* vt) INL {
    const int i = pos_idx(p);
    if (pos_is_s(p)) {
      o.kf[i] = *LDS(bf16x8, kt + (k_lane ^ (32u * i)));
    } else {
      const int h = i / C::DBLK, db = i % C::DBLK;
      const unsigned char* vp = vt + (v_lane ^ (64u * db)) + h * 16 * C::RB;
      const u32x2 v0 = tr_read(vp), v1 = tr_read(vp + 4 * C::RB);
      const u32x4 w = {v0[0], v0[1], v1[0], v1[1]};
      o.vf[i] = __builtin_bit_cast(bf16x8, w);
    }
  };
  auto ktile = [&](auto kst, auto kblk) INL -> const unsigned char* {
    return sp(kst) + decltype(kblk)::value * 32 * C::RB;
  };
  auto vtile = [&](auto vst, auto vblk) INL -> const unsigned char* {
    return sp(vst) + C::TILE + decltype(vblk)::value * 32 * C::RB;
  };

  // One pipeline step: softmax of block u (scores in s_cur, bf16 result to
  // p_cur), S of block u+1 (K tile kt) into s_nxt, and O += V^T P^T of block
  // u-1 (p_prev, V tile vt). Each position issues the LDS reads of the product
  // AHEAD positions later (for the last positions, the first products of the
  // next step, from its tiles nkt / nvt into `nxt`) and forms an equal share
  // of the 16 exponentials. Scheduling fences between positions keep this
  // order, so the matrix core always has the next product queued while the
  // vector unit works on the exponentials.
  auto step = [&](int u, f32x16& s_cur, f32x16& s_nxt, const bf16x8 (&p_prev)[2], bf16x8 (&p_cur)[2], Ops& cur,
                  Ops& nxt, const unsigned char* kt, const unsigned char* vt, const unsigned char* nkt,
                  const unsigned char* nvt, int ld_tile, auto ld_stage, auto ld_part) INL {
    constexpr int LP = decltype(ld_part)::value;   // part of tile ld_tile to load, or -1
    if (masked(u)) apply_mask(u, s_cur);
    constexpr int SPM = 16 / NM;   // exponentials per product
    f32x16 acc = f32x16{};
    float part[4];
    float e_prev = 0.f;
    const float neg_m = -m_ref;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + AHEAD < NM)
        fetch(i + AHEAD, cur, kt, vt);
      else
        fetch(i + AHEAD - NM, nxt, nkt, nvt);
      // This step's share of the ring loads, one load per few products.
      if constexpr (LP >= 0) {
        if (i == 1) issue_load(ld_tile, ld_stage, LP, false);
        if (i == 3) issue_load(ld_tile, ld_stage, LP, true);
      }
      const int k = pos_idx(i);
      if (pos_is_s(i)) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.kf[k], qf[k], acc, 0, 0, 0);
      } else {
        const int h = k / C::DBLK, db = k % C::DBLK;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.vf[k], p_prev[h], oacc[db], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < SPM; ++t) {
        const int r = i * SPM + t;
        const float e = fast_exp2(__builtin_fmaf(s_cur[r], c, neg_m));
        part[r & 3] = r < 4 ? e : part[r & 3] + e;
        if (r & 1) {
          p_cur[r >> 3][(r & 7) - 1] = (__bf16)e_prev;
          p_cur[r >> 3][r & 7] = (__bf16)e;
        }
        e_prev = e;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    s_nxt = acc;
    float sum = (part[0] + part[1]) + (part[2] + part[3]);
    if (__builtin_amdgcn_ballot_w64(!(sum <= kPartMax)) != 0) {
      // Re-base every row of the wave to max(m_ref, row maximum of block u).
      float mx = s_cur[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m_ref, mx * c);
      const float alpha = m_new == -INFINITY ? 0.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) scale_in_place(oacc[db], alpha);
      sum = exps(s_cur, m_ref == -INFINITY ? 0.f : m_ref, p_cur);
    }
    l += sum;
  };

  // Ring bookkeeping before step 2j+1. Tile j+2 must be resident: its K is
  // fetched at the end of step 2j+2. Tile j+3 (issued during steps 2j-1 and
  // 2j) stays in flight. Tile j-1 was last read in step 2j, so after the
  // barrier its stage takes tile j+4, loaded during steps 2j+1 and 2j+2.
  auto tile_sync = [&]() INL {
    __builtin_amdgcn_s_waitcnt(wait_vm(C::LOADS));
    ring_barrier();
  };

  // Prologue: tiles 0..3 in flight, tiles 0 and 1 resident, S of block 0,
  // then step 0 (its product with V is of a zero P against tile 0's V,
  // which is finite).
  issue_tile(0, IC<0>{});
  issue_tile(1, IC<1>{});
  issue_tile(2, IC<2>{});
  issue_tile(3, IC<3>{});
  __builtin_amdgcn_s_waitcnt(wait_vm(2 * C::LOADS));
  ring_barrier();

  f32x16 sa, sb;
  bf16x8 pa[2], pb[2] = {bf16x8{}, bf16x8{}};
  Ops oa, ob;
  {
    bf16x8 kf[C::KSTEPS];
    read_k(IC<0>{}, IC<0>{}, kf);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], acc, 0, 0, 0);
    sa = acc;
  }
#pragma unroll
  for (int p = 0; p < AHEAD; ++p) fetch(p, oa, ktile(IC<0>{}, IC<1>{}), vtile(IC<0>{}, IC<0>{}));
  step(0, sa, sb, pb, pa, oa, ob, ktile(IC<0>{}, IC<1>{}), vtile(IC<0>{}, IC<0>{}), ktile(IC<1>{}, IC<0>{}),
       vtile(IC<0>{}, IC<0>{}), 0, IC<0>{}, IC<-1>{});

  // Steps 1..U, ten per iteration so that every ring stage is a compile-time
  // variable. Step u reads K of block u+1 (tile (u+1)/2) and V of block u-1
  // (tile (u-1)/2). Step U is a drain: its block lies wholly past the last
  // key (non-causal) or above the diagonal (causal), so the mask zeroes its
  // exponentials, and it completes the product of block U-1; the K it reads
  // (and the operands it fetches for a step U+1) are never used.
  // Step u forms S of block u+1, P of block u and the product of block u-1
  // with V; with this wave's last unmasked block wrow0 / 32 (causal), steps
  // from wrow0 / 32 + 2 on add nothing to its rows.
  const int skip_from = wrow0 / 32 + 2;
  auto loads_only = [&](int ld_tile, auto ld_stage, auto ld_part) INL {
    constexpr int LP = decltype(ld_part)::value;
    if constexpr (LP >= 0) {
      issue_load(ld_tile, ld_stage, LP, false);
      issue_load(ld_tile, ld_stage, LP, true);
    }
  };
  auto one = [&](auto s_tag, int u0) INL -> bool {
    constexpr int S = decltype(s_tag)::value;
    const int u = u0 + S;
    const unsigned char* kt = ktile(IC<((S + 2) / 2) % kStages>{}, IC<S % 2>{});
    const unsigned char* vt = vtile(IC<(S / 2) % kStages>{}, IC<S % 2>{});
    const unsigned char* nkt = ktile(IC<((S + 3) / 2) % kStages>{}, IC<(S + 1) % 2>{});
    const unsigned char* nvt = vtile(IC<((S + 1) / 2) % kStages>{}, IC<(S + 1) % 2>{});
    // Tile j+4 (j = (u-1)/2) goes to the stage freed at the last barrier.
    using LST = IC<(S / 2 + 4) % kStages>;
    const int lt = (u - 1) / 2 + 4;
    const bool live = !SKIP || u < skip_from;
    if constexpr (S % 2 == 0) {
      tile_sync();
      if (live)
        step(u, sb, sa, pa, pb, ob, oa, kt, vt, nkt, nvt, lt, LST{}, IC<0>{});
      else
        loads_only(lt, LST{}, IC<0>{});
    } else {
      if (live)
        step(u, sa, sb, pb, pa, oa, ob, kt, vt, nkt, nvt, lt, LST{}, IC<C::LPW == 2 ? 1 : -1>{});
      else
        loads_only(lt, LST{}, IC<C::LPW == 2 ? 1 : -1>{});
    }
    return u == U;
  };
  for (int u0 = 1;; u0 += 2 * kStages) {
    if (one(IC<0>{}, u0)) break;
    if (one(IC<1>{}, u0)) break;
    if (one(IC<2>{}, u0)) break;
    if (one(IC<3>{}, u0)) break;
    if (one(IC<4>{}, u0)) break;
    if (one(IC<5>{}, u0)) break;
    if (one(IC<6>{}, u0)) break;
    if (one(IC<7>{}, u0)) break;
    if (one(IC<8>{}, u0)) break;
    if (one(IC<9>{}, u0)) break;
  }

  // Loads of tiles past the end (zeros, into unread stages) may still be in
  // flight; let them land before the workgroup ends.
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  // Epilogue: O = acc / l, LSE = (m + log2 l) ln 2 in natural-log units.
  const float lt = halves_sum(l);
  const float inv = lt == 0.f ? 0.f : 1.f / lt;
  if (qrow < N) {
    __bf16* og = (__bf16*)a.o + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *(u32x2*)(og + db * 32 + 8 * g + 4 * hh) = w;
      }
    if (hh == 0) a.lse[lse_base + qrow] = lt == 0.f ? -INFINITY : (m_ref + fast_log2(lt)) * kLn2;
  }
  // Every wave is done with the ring before the next item's tiles land in it.
  ring_barrier();
  }
#endif
}

template <int D, int W, bool CAUSAL, bool SKIP>
hipError_t launch(FwdArgs a, int B, int H, hipStream_t s) {
  using C = Cfg<D, W>;
  // Packed variable-length batch: B sequences, tiles of the longest; one
  // workgroup per (sequence, head, tile).
  a.n_qtiles = ((a.cu_seqlens != nullptr ? a.max_seqlen : a.N) + C::BR - 1) / C::BR;
  long long grid = (long long)B * H * a.n_qtiles;
  a.remap = (grid % 8 == 0) ? 1 : 0;
  // Persistent launch: one workgroup per CU (a multiple of 8, one per XCD
  // slot), when there are more items than that and one workgroup fills a CU.
  a.n_items = (int)grid;
  a.persist = 0;
  const int n_cu = cu_count() & ~7;
  if (C::WG_PER_CU == 1 && a.cu_seqlens == nullptr && ((long long)B * H) % 8 == 0 && n_cu >= 8 && grid > n_cu) {
    a.persist = 1;
    grid = n_cu;
  }
  if (a.cu_seqlens != nullptr)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, W, CAUSAL, true, SKIP>), dim3((int)grid), dim3(C::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, W, CAUSAL, false, SKIP>), dim3((int)grid), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

// Causal launches of sequences up to 4096 rows take the SKIP kernel
// (measured: B=4 H=32 N=2048 0.161-0.164 against 0.169 ms, N=4096
// 0.307-0.309 against 0.308-0.315 ms; N=16384 0.2-0.9% slower with it).
template <int D, int W>
hipError_t launch_mask(int causal, const FwdArgs& a, int B, int H, hipStream_t s) {
  if (!causal) return launch<D, W, false, false>(a, B, H, s);
  const int n = a.cu_seqlens != nullptr ? a.max_seqlen : a.N;
  return n <= 4096 ? launch<D, W, true, true>(a, B, H, s) : launch<D, W, true, false>(a, B, H, s);
}

}  // namespace

int cu_count() {
  static int cached[64] = {};   // per device; a racing first lookup writes the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

hipError_t launch_fwd_bf16(int d, int causal, FwdArgs a, int B, int H, hipStream_t s) {
  // The kernel needs c > 0 so that -inf scores stay -inf after scaling; a
  // zero scale becomes the smallest normal float, whose products with any
  // finite score round exp2 to 1 exactly as scale 0 would.
  a.c = fmaxf(a.c, FLT_MIN);
  if (d == 64) {
    // Up to four 256-row items per CU, 128-row workgroups two to a CU
    // (measured: B=8 H=12 N=1024 0.043 against 0.048 ms, B=2 H=32 N=4096
    // causal 0.184 against 0.188 ms); beyond that the persistent 256-row
    // launch (N=16384: 1.12 against 1.15 ms).
    const long long items256 = (long long)B * H * (((a.cu_seqlens != nullptr ? a.max_seqlen : a.N) + 255) / 256);
    if (items256 <= 4LL * cu_count()) return launch_mask<64, 4>(causal, a, B, H, s);
    return launch_mask<64, 8>(causal, a, B, H, s);
  }
  return launch_mask<128, 8>(causal, a, B, H, s);
}

}  // namespace fa
