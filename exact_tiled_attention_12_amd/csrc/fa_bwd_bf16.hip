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
//   * one workgroup (4 waves) per (batch, head, 256-key tile); each wave owns
//     64 keys (two 32-key blocks); the dK and dV accumulators of those keys
//     (2 x 64 x d floats) stay in registers for the whole pass, and V of the
//     wave's keys is held as MFMA operands;
//   * the workgroup's K tile sits in LDS for the whole pass; query tiles of 32
//     rows (Q, dO, L, D) stream through a 2-stage LDS ring with HBM->LDS
//     buffer loads, one barrier per tile;
//   * S = Q K^T and dP = dO V^T are formed with lanes = keys (Q and dO rows
//     read in a permuted order), so the exponentiated P and dS come out in the
//     operand layout of dV = P^T dO and dK = dS^T Q; the other orientation of
//     Q and dO is read straight from the row-major tiles with
//     ds_read_b64_tr_b16;
//   * dS is written to LDS once (transposed, 16-byte writes) and dQ of tile
//     i-1 is formed while tile i is processed: each wave takes one 32-column
//     slice of dQ over all 256 keys (lanes = d) and adds it atomically;
//   * rows of the LDS tiles are XOR-swizzled per 16-byte chunk so that both
//     the 16-row reads and the 4-row transposed reads hit distinct banks.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKW = 64;              // keys per wave
constexpr int kBC = kKW * kWaves;    // keys per workgroup
constexpr int kBR = 32;              // query rows per tile

#define LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

template <int D>
struct Cfg {
  static constexpr int RB = 2 * D;                   // bytes per row
  static constexpr int CPR = RB / 16;                // 16-byte chunks per row
  static constexpr int K_BYTES = kBC * RB;           // the workgroup's K tile
  static constexpr int QT = kBR * RB;                // one Q or dO tile
  static constexpr int STAGE = 2 * QT + 2 * kBR * 4; // Q, dO, L, D
  static constexpr int DS_BYTES = kBC * kBR * 2;     // dS^T tile [key][q]
  static constexpr int OFF_K = 0;
  static constexpr int OFF_DS = OFF_K + K_BYTES;
  static constexpr int OFF_RING = OFF_DS + 2 * DS_BYTES;
  static constexpr int LDS_BYTES = OFF_RING + 2 * STAGE;
  static constexpr int RPL = 1024 / RB;              // rows per 1 KiB wave-load
  static constexpr int K_LOADS = K_BYTES / 1024 / kWaves;
  static constexpr int QT_LOADS = QT / 1024 / kWaves;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static_assert(QT_LOADS >= 1 && K_LOADS >= 1, "tile split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
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

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_bf16_kernel(BwdArgs a) {
  // Device pass only (the host pass needs just the launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg<D>;
  // The K tile, the dS^T buffers and the query-tile ring are separate
  // variables: while the next query tile is in flight into the ring only the
  // K tile and dS^T are read, so the compiler needs no wait on the load.
  __shared__ __attribute__((aligned(1024))) unsigned char kt_s[C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char ds_s[2 * C::DS_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char rg_s[2 * C::STAGE];
  auto ring = [&](int st) -> unsigned char* { return rg_s + st * C::STAGE; };
  auto dsb = [&](int st) -> unsigned char* { return ds_s + st * C::DS_BYTES; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int ts = j16 >> 2, tq = j16 & 3;     // transposed-read source row / column group

  int wg = blockIdx.x;
  if (a.remap) wg = xcd_remap(wg, gridDim.x);
  const int bh = wg / a.n_tiles;
  const int kt = wg - bh * a.n_tiles;        // key tile; tile 0 (heaviest when causal) first
  const int N = a.N;
  const size_t base = (size_t)bh * (size_t)N * D;
  const unsigned head_bytes = (unsigned)N * C::RB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const __bf16*)a.q + base, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const __bf16*)a.k + base, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const __bf16*)a.v + base, head_bytes);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc((const __bf16*)a.dout + base, head_bytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse + (size_t)bh * N, (unsigned)N * 4);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dvec + (size_t)bh * N, (unsigned)N * 4);
  float* __restrict__ dQg = a.dq_acc + base;

  const int k0 = kt * kBC;
  const int kw0 = k0 + wave * kKW;

  // ---- HBM -> LDS loads (rows past N read as zero).
  auto load_rows = [&](const __amdgpu_buffer_rsrc_t& r, unsigned char* dst, int row0, int t) {
    const int row = t * C::RPL + lane / C::CPR;
    const int p = lane % C::CPR;
    const unsigned g = (unsigned)(row0 + row) * C::RB + 16 * (p ^ swz<D>(row));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS(void, dst + t * 1024), 16, g, 0, 0, 0);
  };
  auto issue_qtile = [&](int qt, int st) {
    unsigned char* so = ring(st);
#pragma unroll
    for (int i = 0; i < C::QT_LOADS; ++i) {
      const int t = wave * C::QT_LOADS + i;
      load_rows(rq, so, qt * kBR, t);
      load_rows(rg, so + C::QT, qt * kBR, t);
    }
    if (wave == 0) {
      // L and D of the tile's 32 rows: 8 lanes x 16 bytes each.
      if (lane < 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, LDS(void, so + 2 * C::QT), 16,
                                                 (unsigned)(qt * kBR) * 4 + 16 * lane, 0, 0, 0);
      else if (lane < 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, LDS(void, so + 2 * C::QT), 16,
                                                 (unsigned)(qt * kBR) * 4 + 16 * (lane - 8), 0, 0, 0);
    }
  };

  const int n_qt = (N + kBR - 1) / kBR;
  const int qt_begin = CAUSAL ? k0 / kBR : 0;

  // K tile (whole workgroup) and the first query tile.
#pragma unroll
  for (int i = 0; i < C::K_LOADS; ++i) load_rows(rk, kt_s, k0, wave * C::K_LOADS + i);
  if (qt_begin < n_qt) issue_qtile(qt_begin, 0);

  // V rows of the wave's keys as the B operand of dP = dO V^T (lanes = keys).
  bf16x8 vf[2][C::KSTEPS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const unsigned off = (unsigned)(kw0 + kb * 32 + l32) * C::RB + kk * 32 + hh * 16;
      vf[kb][kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }

  // ---- per-lane LDS addresses (byte offsets; chunk bits XORed per step).
  // Rows of a 32-row block read with lanes = one row each (Q, dO: permuted).
  const int prow = acc_row_to_key(l32);
  const int fq = swz<D>(prow);
  const unsigned a_lane = (unsigned)prow * C::RB + 16 * ((hh ^ fq) & 1) + 32 * (fq >> 1);
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

  f32x16 dk[2][C::DBLK], dv[2][C::DBLK];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
      dk[kb][db] = f32x16{};
      dv[kb][db] = f32x16{};
    }
  const float c = a.c;

  // dQ of the tile whose dS^T sits in dS buffer `st`: this wave's 32
  // columns (D = 64: two waves per column block, each over half of the keys).
  // Operand reads run one 16-key step ahead of the MFMAs.
  auto dq_tile = [&](int qt, int st) {
    const int q0 = qt * kBR;
    int kc_end = kBC / 16;
    if (CAUSAL) kc_end = min(kc_end, (q0 + kBR - 1 - k0) / 16 + 1);
    const int db = D == 128 ? wave : (wave & 1);
    const int kc0 = D == 128 ? 0 : (wave >> 1) * 8;
    const int kc1 = D == 128 ? kc_end : min(kc_end, kc0 + 8);
    const unsigned char* sb = dsb(st);
    const unsigned char* s0a = sb + s_lane[0];
    const unsigned char* s1a = sb + s_lane[1];
    const unsigned char* k0a = kt_s + (t_lane[0] ^ (64u * db));
    const unsigned char* k1a = kt_s + (t_lane[1] ^ (64u * db));
    auto rd = [&](int kc) {
      Tr4 t;
      t.v[0] = tr_read(s0a + kc * 16 * 64);
      t.v[1] = tr_read(s1a + kc * 16 * 64);
      t.v[2] = tr_read(k0a + kc * 16 * C::RB);
      t.v[3] = tr_read(k1a + kc * 16 * C::RB);
      return t;
    };
    f32x16 acc = f32x16{};
    if (kc0 < kc1) {
      Tr4 cur = rd(kc0);
      for (int kc = kc0; kc < kc1; ++kc) {
        Tr4 nxt = cur;
        if (kc + 1 < kc1) nxt = rd(kc + 1);
        __builtin_amdgcn_sched_barrier(0);
        acc = mma(join(cur.v[0], cur.v[1]), join(cur.v[2], cur.v[3]), acc);
        cur = nxt;
      }
      const int d = db * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (q < N) unsafeAtomicAdd(dQg + (size_t)q * D + d, acc[r]);
      }
    }
  };

  // One query tile of this wave's 64 keys: S, dP, P, dS, dV, dK; dS^T to LDS.
  // Q, dO, L, D come from ring stage `st`, dS^T goes to dS buffer `st`.
  auto key_tile = [&](int qt, int st, bool mask, bool act) {
    const int q0 = qt * kBR;
    const unsigned char* qs = ring(st);
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    // Operand reads run one d-step ahead of the MFMAs (double buffer); the
    // scheduling fences keep the compiler from hoisting every read at once.
    bf16x8 fq[2], fg[2], fk0[2], fk1[2];
    auto rd = [&](int kk, int b) {
      fq[b] = *LDS(bf16x8, qs + (a_lane ^ (32u * kk)));
      fg[b] = *LDS(bf16x8, qs + C::QT + (a_lane ^ (32u * kk)));
      fk0[b] = *LDS(bf16x8, kt_s + (k_lane ^ (32u * kk)));
      fk1[b] = *LDS(bf16x8, kt_s + (k_lane ^ (32u * kk)) + 32 * C::RB);
    };
    rd(0, 0);
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const int b = kk & 1;
      if (kk + 1 < C::KSTEPS) rd(kk + 1, b ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      s[0] = mma(fq[b], fk0[b], s[0]);
      dp[0] = mma(fg[b], vf[0][kk], dp[0]);
      s[1] = mma(fq[b], fk1[b], s[1]);
      dp[1] = mma(fg[b], vf[1][kk], dp[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P = exp2(S c - L log2 e), dS = P (dP - D) at the 16 rows this lane
    // holds. Entry (q0 + ql, key) is kept iff ql >= lim; on tiles that need
    // no mask lim is below every ql, so one code path serves both.
    const float* Ls = (const float*)(qs + 2 * C::QT);
    const float* Ds = Ls + kBR;
    bf16x8 pf[2][2], df[2][2];
    int lim[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kw0 + kb * 32 + l32;
      lim[kb] = !mask ? -1 : (!act || key >= N) ? kBR : CAUSAL ? key - q0 : -1;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ql = slot_key(r, hh);
      const float l2 = Ls[ql] * kLog2e, dd = Ds[ql];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -l2));
        p = ql >= lim[kb] ? p : 0.f;
        const float ds = p * (dp[kb][r] - dd);
        pf[kb][r >> 3][r & 7] = (__bf16)p;
        df[kb][r >> 3][r & 7] = (__bf16)ds;
      }
    }
    // dV += P^T dO, dK += dS^T Q: B operands read transposed from the tiles,
    // one (ks, db) step ahead of the MFMAs.
    auto trd = [&](int step) {
      const int ks = step / C::DBLK, db = step % C::DBLK;
      const unsigned char* ko = qs + ks * 16 * C::RB;
      Tr4 t;
      t.v[0] = tr_read(ko + C::QT + (t_lane[0] ^ (64u * db)));
      t.v[1] = tr_read(ko + C::QT + (t_lane[1] ^ (64u * db)));
      t.v[2] = tr_read(ko + (t_lane[0] ^ (64u * db)));
      t.v[3] = tr_read(ko + (t_lane[1] ^ (64u * db)));
      return t;
    };
    __builtin_amdgcn_sched_barrier(0);
    Tr4 cur = trd(0);
#pragma unroll
    for (int step = 0; step < 2 * C::DBLK; ++step) {
      const int ks = step / C::DBLK, db = step % C::DBLK;
      Tr4 nxt = cur;
      if (step + 1 < 2 * C::DBLK) nxt = trd(step + 1);
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 gb = join(cur.v[0], cur.v[1]), qb = join(cur.v[2], cur.v[3]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dv[kb][db] = mma(pf[kb][ks], gb, dv[kb][db]);
        dk[kb][db] = mma(df[kb][ks], qb, dk[kb][db]);
      }
      cur = nxt;
      __builtin_amdgcn_sched_barrier(0);
    }
    // dS^T rows (keys) of this wave: 8 queries per 16-byte write.
    unsigned char* sp = dsb(st) + w_lane;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        *LDS(bf16x8, sp + kb * 32 * 64 + 16 * ((2 * ks + hh) ^ wsw)) = df[kb][ks];
  };

  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): K tile, first query tile, V operands
  __syncthreads();

  // Query tile qt (i = qt - qt_begin) uses ring stage and dS buffer i % 2.
  // After the barrier tile qt is resident and dS^T of tile qt-1 complete; the
  // tile's own work reads the ring, then the load of tile qt+1 is queued into
  // the other stage (free: its last reader was tile qt-1) and overlaps the dQ
  // of tile qt-1, which reads only the K tile and dS^T.
  for (int qt = qt_begin; qt < n_qt; ++qt) {
    const int i = qt - qt_begin, st = i & 1;
    if (i > 0) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's load of tile qt and its dQ atomics
      __syncthreads();
    }
    // Waves whose keys all follow the tile's rows run the tile fully masked
    // (one straight-line path keeps the accumulators in registers).
    const int q0 = qt * kBR;
    const bool active = !CAUSAL || kw0 <= q0 + kBR - 1;
    const bool mask = !active || kw0 + kKW > N || (CAUSAL && kw0 + kKW - 1 > q0);
    key_tile(qt, st, mask, active);
    if (qt + 1 < n_qt) issue_qtile(qt + 1, st ^ 1);
    if (i > 0) dq_tile(qt - 1, st ^ 1);
  }
  if (qt_begin < n_qt) {
    __syncthreads();
    dq_tile(n_qt - 1, (n_qt - 1 - qt_begin) & 1);
  }

  // Epilogue: dK = scale * acc, dV = acc (lanes = d, rows = keys); rows past N dropped.
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
#endif
}

}  // namespace

hipError_t launch_bwd_bf16_main(int d, int causal, BwdArgs a, int B, int H, hipStream_t s) {
  a.n_tiles = (a.N + kBC - 1) / kBC;
  const long long grid = (long long)B * H * a.n_tiles;
  a.remap = grid % 8 == 0 ? 1 : 0;
  if (d == 64) {
    if (causal) hipLaunchKernelGGL((bwd_bf16_kernel<64, true>), dim3(grid), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((bwd_bf16_kernel<64, false>), dim3(grid), dim3(kThreads), 0, s, a);
  } else {
    if (causal) hipLaunchKernelGGL((bwd_bf16_kernel<128, true>), dim3(grid), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((bwd_bf16_kernel<128, false>), dim3(grid), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace fa
