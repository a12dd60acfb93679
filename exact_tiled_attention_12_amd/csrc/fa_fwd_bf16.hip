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
//     groups the tiles of a (batch, head) on one XCD;
//   * K and V tiles of 64 keys move from HBM straight into a 3-stage LDS ring
//     (buffer loads with an LDS destination; rows past N read as zero), two
//     tiles ahead of use, with one workgroup barrier per tile;
//   * S^T = K Q^T and O^T = V^T P^T on the 32x32x16 bf16 MFMA: K rows are read
//     in a permuted order so every lane owns one query and holds its
//     exponentiated scores in exactly the operand layout of the second
//     product; V stays row-major in LDS and is read transposed with
//     ds_read_b64_tr_b16;
//   * within a wave the loop is software-pipelined: the QK^T products of tile
//     j+1 are issued while the softmax of tile j runs;
//   * the running maximum is re-based only when it grows by more than
//     tau = 8 (log2 units) on some row of the wave ("FlashAttention v1～v4
//     完整进化史", v4 part 3); until then exponentials are taken against the
//     stale maximum (they stay below 2^8), and O / l is exact at the end;
//   * LDS rows are XOR-swizzled per 16-byte chunk so the K reads (16 rows, one
//     chunk) and the transposed V reads (4 rows x 4 chunks) are free of bank
//     conflicts.
#include <cfloat>
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;   // query rows per workgroup
constexpr int kBC = 64;            // keys per tile
constexpr int kStages = 3;
constexpr float kTau = 8.f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

template <int D>
struct Cfg {
  static constexpr int RB = D * 2;                  // bytes per row
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row
  static constexpr int TILE = kBC * RB;             // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int LDS_BYTES = kStages * STAGE;   // three __shared__ stages
  static constexpr int LPW = TILE / 1024 / kWaves;  // 1 KiB wave-loads per wave per tensor
  static constexpr int RPL = 1024 / RB;             // rows per wave-load
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static_assert(LPW >= 1 && LPW * kWaves * 1024 == TILE, "tile split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  // The body is compiled in the device pass only: the host pass needs just the
  // launch stub, and its front end drops the stub of a kernel whose lambdas
  // capture buffer resources.
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg<D>;
  // One variable per ring stage: with the stage known at compile time the
  // compiler can tell a tile being read from the tile being loaded, and needs
  // no wait on the in-flight loads before the reads.
  __shared__ __attribute__((aligned(1024))) unsigned char st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[C::STAGE];
  auto sp = [&](auto stag) -> unsigned char* {
    constexpr int S = decltype(stag)::value;
    if constexpr (S == 0) return st0;
    else if constexpr (S == 1) return st1;
    else return st2;
  };

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
  const size_t base = (size_t)bh * (size_t)N * D;
  const unsigned head_bytes = (unsigned)N * C::RB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const __bf16*)a.q + base, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const __bf16*)a.k + base, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const __bf16*)a.v + base, head_bytes);

  const int q0 = qt * kBR;
  const int wrow0 = q0 + wave * 32;
  const int qrow = wrow0 + l32;

  const int n_kv = (N + kBC - 1) / kBC;
  const int kv_end = CAUSAL ? min(n_kv, (min(q0 + kBR, N) - 1) / kBC + 1) : n_kv;

  // --- tile loads: HBM -> LDS, no registers. Wave-load t covers rows
  // [t*RPL, t*RPL+RPL) of the tile; lane l fills physical chunk l % CPR of
  // row t*RPL + l / CPR with the logical chunk that the swizzle maps there.
  auto issue_tile = [&](int j, auto stag) __device__ {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int tl = wave * C::LPW + i;
      const int row = tl * C::RPL + lane / C::CPR;
      const int p = lane % C::CPR;
      const unsigned grow = (unsigned)(j * kBC + row) * C::RB;
      unsigned char* kd = sp(stag) + tl * 1024;
      unsigned char* vd = kd + C::TILE;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, LDS(void, kd), 16, grow + 16 * (p ^ k_swz<D>(row)), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, LDS(void, vd), 16, grow + 16 * (p ^ v_swz<D>(row)), 0, 0, 0);
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

  // S^T of one 32-key block (blk) of the tile in stage `stag`.
  auto qk = [&](auto stag, int blk, f32x16& s) __device__ {
    const unsigned char* kt = sp(stag);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const unsigned addr = (k_lane ^ (32u * kk)) + blk * 32 * C::RB;
      const bf16x8 af = *LDS(bf16x8, kt + addr);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[kk], acc, 0, 0, 0);
    }
    s = acc;
  };

  // Softmax of one 32-key block against the reference maximum, then
  // O += V^T P^T over its 32 keys. `mask` applies key < N and the causal
  // condition on ragged and diagonal blocks; a block above the diagonal of
  // every row of the wave comes out fully masked and adds nothing. c > 0
  // (the launcher clamps it), so masked scores stay -inf through the scaling.
  auto softmax_pv = [&](bool mask, int u, f32x16& s, auto stag, int blk) __device__ {
    if (mask) {
      const int key0 = u * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + slot_key(r, hh);
        const bool ok = key < N && (!CAUSAL || key <= qrow);
        s[r] = ok ? s[r] : -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = halves_max(mx);
    const float mxs = mx * c;
    // Re-base only when the maximum grew by more than tau on some row of the
    // wave (a wave-uniform decision). The accumulator is then scaled inside
    // the first product of this block on one branch and fed unchanged on the
    // other, so both branches end in a matrix-core write of the same
    // registers and the untaken path costs no copies.
    const bool grow = __builtin_amdgcn_ballot_w64(mxs > m_ref + kTau) != 0;
    const float m_new = grow ? fmaxf(m_ref, mxs) : m_ref;
    const float alpha = (!grow || m_new == -INFINITY) ? 1.f : fast_exp2(m_ref - m_new);
    m_ref = m_new;
    l *= alpha;
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    bf16x8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(__builtin_fmaf(s[r], c, -m_use));
      part[r & 3] += e;
      pf[r >> 3][r & 7] = (__bf16)e;
    }
    l += (part[0] + part[1]) + (part[2] + part[3]);
    // V tile of `stage`, 16-key half ks of block blk: the key offset is a
    // compile-time immediate once blk and ks are.
    const unsigned char* vt = sp(stag) + C::TILE;
    auto read_v = [&](auto ofs_tag, bf16x8 (&vf)[C::DBLK]) __device__ {
      constexpr int OFS = decltype(ofs_tag)::value;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) {
        const unsigned char* vp = vt + (v_lane ^ (64u * db)) + OFS;
        const u32x2 v0 = tr_read(vp), v1 = tr_read(vp + 4 * C::RB);
        const u32x4 w = {v0[0], v0[1], v1[0], v1[1]};
        vf[db] = __builtin_bit_cast(bf16x8, w);
      }
    };
    if (grow) {
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) scale_in_place(oacc[db], alpha);
    }
    auto pv = [&](auto ofs0, auto ofs1) __device__ {
      bf16x8 vf[C::DBLK];
      read_v(ofs0, vf);
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pf[0], oacc[db], 0, 0, 0);
      read_v(ofs1, vf);
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pf[1], oacc[db], 0, 0, 0);
    };
    if (blk == 0)
      pv(std::integral_constant<int, 0>{}, std::integral_constant<int, 16 * C::RB>{});
    else
      pv(std::integral_constant<int, 32 * C::RB>{}, std::integral_constant<int, 48 * C::RB>{});
  };

  // 32-key blocks: u = 2*tile + blk. Every wave runs every block of the
  // workgroup's tiles (no divergent skips: they would make the accumulators
  // change registers between branches); masking is needed on ragged and
  // diagonal blocks, and blocks past a wave's last row are fully masked.
  auto masked = [&](int u) __device__ { return u * 32 + 32 > N || (CAUSAL && u * 32 + 31 > wrow0); };
  auto block = [&](int u, f32x16& cur, f32x16& nxt, auto stag, int blk, auto nstag, int nblk) __device__ {
    if (u + 1 < 2 * kv_end) qk(nstag, nblk, nxt);
    softmax_pv(masked(u), u, cur, stag, blk);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  // Prologue: tiles 0 and 1 in flight, S of block 0.
  issue_tile(0, I0{});
  if (kv_end > 1) issue_tile(1, I1{});
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  f32x16 sa, sb;
  qk(I0{}, 0, sa);

  // Tile j (in stage j % 3): blocks 2j (S in sa) and 2j+1; the next block's
  // QK^T is issued alongside each softmax. The barrier makes tile j+1
  // resident and frees the stage of tile j-1 for tile j+2. The loop is
  // unrolled by the ring depth so every stage is a compile-time variable.
  auto tile = [&](int j, auto stag) __device__ {
    constexpr int S = decltype(stag)::value;
    using S1 = std::integral_constant<int, (S + 1) % kStages>;
    using S2 = std::integral_constant<int, (S + 2) % kStages>;
    if (j > 0) {
      // The compiler does not order LDS-destination loads before a barrier by
      // itself: wait for this wave's loads of tile j+1 (the only ones in
      // flight), then the barrier publishes every wave's part.
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    }
    if (j + 2 < kv_end) issue_tile(j + 2, S2{});
    block(2 * j, sa, sb, stag, 0, stag, 1);
    block(2 * j + 1, sb, sa, stag, 1, S1{}, 0);
  };
  int j = 0;
  for (; j + kStages <= kv_end; j += kStages) {
    tile(j, I0{});
    tile(j + 1, I1{});
    tile(j + 2, I2{});
  }
  if (j < kv_end) tile(j, I0{});
  if (j + 1 < kv_end) tile(j + 1, I1{});

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
    if (hh == 0) a.lse[(size_t)bh * N + qrow] = lt == 0.f ? -INFINITY : (m_ref + fast_log2(lt)) * kLn2;
  }
#endif
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(int d, int causal, FwdArgs a, int B, int H, hipStream_t s) {
  // The kernel needs c > 0 so that -inf scores stay -inf after scaling; a
  // zero scale becomes the smallest normal float, whose products with any
  // finite score round exp2 to 1 exactly as scale 0 would.
  a.c = fmaxf(a.c, FLT_MIN);
  a.n_qtiles = (a.N + kBR - 1) / kBR;
  const long long grid = (long long)B * H * a.n_qtiles;
  a.remap = (grid % 8 == 0) ? 1 : 0;
  if (d == 64) return causal ? launch<64, true>(a, (int)grid, s) : launch<64, false>(a, (int)grid, s);
  return causal ? launch<128, true>(a, (int)grid, s) : launch<128, false>(a, (int)grid, s);
}

}  // namespace fa
