// Recompute-based attention backward for gfx950: the preprocess and finish
// passes (both types) and the float32 main kernel; the bf16 main kernel is in
// fa_bwd_bf16.hip.
//
// What it computes ("6.1 FlashAttention V1详解", sections 6.1-6.2;
// "FlashAttention v1～v4 完整进化史", v2 part 1 and v4 part 4): S and P are
// not stored by the forward; here P = exp(S - L) is recomputed tile by tile
// from Q, K and the saved log-sum-exp L, and
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dK = scale dS^T Q,  dQ = scale dS K      (five matrix products per tile).
// dQ is summed across key tiles with float32 atomics (the pages' dQ atomics),
// or, in the bf16 fixed-order mode, in ascending key-tile order.
//
// Three launches:
//   1. preprocess: D_i = sum_c dO_ic O_ic (float32) and zero the float32 dQ
//      accumulator;
//   2. main: one workgroup (4 waves) per (batch, head, 128-key tile); each
//      wave owns 32 keys, keeps its K and V operand fragments and its dK, dV
//      accumulators in registers, and walks the query tiles whose rows reach
//      its keys (causal: the tiles at or below the diagonal). Per query tile
//      the workgroup stages Q and dO in LDS in both orientations, and
//      S^T-style products (lanes = keys) give P and dS already in the operand
//      layout of dV = P^T dO and dK = dS^T Q. dS goes through LDS once so
//      dQ = dS K can be formed with lanes = d and added atomically;
//   3. finish: dQ = scale * accumulator, cast to the output type.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBC = 128;     // keys per workgroup (4 waves x 32)

template <class Tr, int D>
struct BwdCfg {
  using T = typename Tr::T;
  static constexpr int QB = sizeof(T) == 2 ? 2 : 1;   // 32-row query blocks per tile
  static constexpr int BR = 32 * QB;                  // query rows per tile
  static constexpr int E = 16 / sizeof(T);
  static constexpr int KTs = kBC + E;                 // K^T  [D][kBC]
  static constexpr int QSs = D + E;                   // Q, dO row-major [BR][D]
  static constexpr int QTs = BR + E;                  // Q^T, dO^T [D][BR]
  static constexpr int DSs = kBC + E;                 // dS   [BR][kBC]
  static constexpr int KT_OFF = 0;
  static constexpr int QS_OFF = KT_OFF + D * KTs;
  static constexpr int QT_OFF = QS_OFF + BR * QSs;
  static constexpr int OS_OFF = QT_OFF + D * QTs;
  static constexpr int OT_OFF = OS_OFF + BR * QSs;
  static constexpr int DS_OFF = OT_OFF + D * QTs;
  static constexpr int T_ELEMS = DS_OFF + BR * DSs;
  static constexpr int LDS_BYTES = T_ELEMS * (int)sizeof(T) + 2 * BR * 4;
  static constexpr int CPR = D / E;                   // 16-byte chunks per row
  static constexpr int QVG = kThreads / CPR;          // row groups for a BR x D tile
  static constexpr int QKPT = BR / QVG;               // rows per thread (BR x D tile)
  static constexpr int KVG = kThreads / CPR;
  static constexpr int KKPT = kBC / KVG;              // rows per thread (kBC x D tile)
  static constexpr int KSTEPS = D / (2 * Tr::KPL);
  static constexpr int PSTEPS = 32 / (2 * Tr::KPL);
  static constexpr int CSTEPS = kBC / (2 * Tr::KPL);  // steps over the workgroup's keys
  static constexpr int DBLK = D / 32;
  static_assert(QKPT * QVG == BR && KKPT * KVG == kBC, "tile split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// ---------------------------------------------------------------- preprocess
template <class Tr, int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdArgs a, long long rows) {
  using T = typename Tr::T;
  constexpr int E = 16 / sizeof(T);
  constexpr int CPR = D / E;
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = gid / CPR;
  const int chunk = (int)(gid % CPR);
  float part = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + chunk * E;
    const u32x4 ov = *(const u32x4*)((const T*)a.o + off);
    const u32x4 gv = *(const u32x4*)((const T*)a.dout + off);
    const T* op = (const T*)&ov;
    const T* gp = (const T*)&gv;
#pragma unroll
    for (int e = 0; e < E; ++e) part += (float)op[e] * (float)gp[e];
    float* acc = a.dq_acc + off;
#pragma unroll
    for (int e = 0; e < E; e += 4) *(f32x4*)(acc + e) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Fixed-order mode: clear the per-tile counters and the error flag.
  if (a.dq_cnt != nullptr && gid < a.n_cnt) a.dq_cnt[gid] = 0;
  // Sum over the CPR consecutive lanes that hold one row (CPR divides 64).
#pragma unroll
  for (int sh = 1; sh < CPR; sh <<= 1) part += __shfl_xor(part, sh, 64);
  if (row < rows && chunk == 0) a.dvec[row] = part;
}

// ---------------------------------------------------------------- finish
template <class Tr, int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdArgs a, long long n4) {
  using T = typename Tr::T;
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n4) return;
  f32x4 v = *(const f32x4*)(a.dq_acc + 4 * i) * a.scale;
  // Fixed-order mode: a wait that ran out left the order (and maybe the
  // sum) unknown; dq becomes NaN so that the failure cannot pass unseen.
  if (a.dq_err != nullptr && *(const volatile int*)a.dq_err != 0) v = f32x4{NAN, NAN, NAN, NAN};
  T* dst = (T*)a.dq + 4 * i;
  if constexpr (sizeof(T) == 2) {
    u32x2 w;
    w[0] = pack_bf16x2(v[0], v[1]);
    w[1] = pack_bf16x2(v[2], v[3]);
    *(u32x2*)dst = w;
  } else {
    *(f32x4*)dst = v;
  }
}

// ------------------------------------- grouped-query dK, dV chunk sum
// dk, dv [B, H_kv, N, d] = sum over the group's query heads c = 0, 1, ... (in
// that order) of their float32 dK (already scaled) and dV, rounded to bf16.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkv_sum_kernel(BwdArgs a, long long n4) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n4) return;
  const long long e = 4 * i;                          // element of [B H_kv][N][d]
  const long long per_head = (long long)a.N * D;
  const long long bh = e / per_head, in_head = e - bh * per_head;
  const int C = a.group;
  const float* pk = a.dkv_part + (size_t)bh * C * per_head + in_head;
  const float* pv = pk + (size_t)n4 * 4 * C;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < C; ++c) {
    sk += __builtin_nontemporal_load((const f32x4*)(pk + (size_t)c * per_head));
    sv += __builtin_nontemporal_load((const f32x4*)(pv + (size_t)c * per_head));
  }
  u32x2 w;
  w[0] = pack_bf16x2(sk[0], sk[1]);
  w[1] = pack_bf16x2(sk[2], sk[3]);
  *(u32x2*)((__bf16*)a.dk + e) = w;
  w[0] = pack_bf16x2(sv[0], sv[1]);
  w[1] = pack_bf16x2(sv[2], sv[3]);
  *(u32x2*)((__bf16*)a.dv + e) = w;
}

// ---------------------------------------------------------------- main
template <class Tr, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(BwdArgs a) {
  using C = BwdCfg<Tr, D>;
  using T = typename Tr::T;
  using Frag = typename Tr::Frag;
  constexpr int KPL = Tr::KPL;
  constexpr int BR = C::BR;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[C::LDS_BYTES];
  T* lds = (T*)smem_raw;
  T* KT = lds + C::KT_OFF;
  T* QS = lds + C::QS_OFF;
  T* QT = lds + C::QT_OFF;
  T* OS = lds + C::OS_OFF;
  T* OT = lds + C::OT_OFF;
  T* DS = lds + C::DS_OFF;
  float* LS = (float*)(lds + C::T_ELEMS);   // LSE * log2(e) of the tile's rows
  float* DD = LS + BR;                       // D of the tile's rows

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  int wg = blockIdx.x;
  if (a.remap) wg = xcd_remap(wg, gridDim.x);
  const int bh = wg / a.n_tiles;
  const int kt = wg - bh * a.n_tiles;         // key tile; tile 0 (the heaviest when causal) first
  const int N = a.N;
  const size_t base = (size_t)bh * (size_t)N * D;
  const T* __restrict__ Qg = (const T*)a.q + base;
  const T* __restrict__ Kg = (const T*)a.k + base;
  const T* __restrict__ Vg = (const T*)a.v + base;
  const T* __restrict__ Gg = (const T*)a.dout + base;
  const float* __restrict__ Lg = a.lse + (size_t)bh * N;
  const float* __restrict__ Dg = a.dvec + (size_t)bh * N;
  float* __restrict__ dQg = a.dq_acc + base;

  const int k0 = kt * kBC;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;                  // this lane's key
  const bool key_ok = key < N;

  // K and V rows of this lane's key as operands (B of S = Q K^T and of dP = dO V^T).
  Frag kf[C::KSTEPS], vf[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
    const size_t off = (size_t)key * D + kk * 2 * KPL + hh * KPL;
    kf[kk] = key_ok ? Tr::load(Kg + off) : Tr::zero();
    vf[kk] = key_ok ? Tr::load(Vg + off) : Tr::zero();
  }
  // K^T of the workgroup's keys in LDS (operand of dQ = dS K).
  {
    const int c = tid % C::CPR, g = tid / C::CPR;
    u32x4 r[C::KKPT];
#pragma unroll
    for (int i = 0; i < C::KKPT; ++i) {
      const int kr = k0 + g * C::KKPT + i;
      r[i] = kr < N ? *(const u32x4*)(Kg + (size_t)kr * D + c * C::E) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int e = 0; e < C::E; ++e) {
      T tmp[C::KKPT];
#pragma unroll
      for (int i = 0; i < C::KKPT; ++i) tmp[i] = ((const T*)&r[i])[e];
      store_bytes<C::KKPT * (int)sizeof(T)>(KT + (c * C::E + e) * C::KTs + g * C::KKPT, tmp);
    }
  }

  const int n_qt = (N + BR - 1) / BR;
  const int qt_begin = CAUSAL ? k0 / BR : 0;

  // Global -> register stage of one query tile (Q, dO, L, D), then -> LDS.
  const int sc = tid % C::CPR, sg = tid / C::CPR;
  u32x4 qreg[C::QKPT], greg[C::QKPT];
  float lreg = 0.f, dreg = 0.f;
  auto gload = [&](int qt) {
    const int r0 = qt * BR;
#pragma unroll
    for (int i = 0; i < C::QKPT; ++i) {
      const int r = r0 + sg * C::QKPT + i;
      const bool ok = r < N;
      qreg[i] = ok ? *(const u32x4*)(Qg + (size_t)r * D + sc * C::E) : u32x4{0, 0, 0, 0};
      greg[i] = ok ? *(const u32x4*)(Gg + (size_t)r * D + sc * C::E) : u32x4{0, 0, 0, 0};
    }
    if (tid < BR) {
      const int r = r0 + tid;
      // Rows past N get L = +inf so their recomputed P is 0.
      lreg = r < N ? Lg[r] * kLog2e : INFINITY;
      dreg = r < N ? Dg[r] : 0.f;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < C::QKPT; ++i) {
      const int rl = sg * C::QKPT + i;
      *(u32x4*)(QS + rl * C::QSs + sc * C::E) = qreg[i];
      *(u32x4*)(OS + rl * C::QSs + sc * C::E) = greg[i];
    }
#pragma unroll
    for (int e = 0; e < C::E; ++e) {
      T tq[C::QKPT], tg[C::QKPT];
#pragma unroll
      for (int i = 0; i < C::QKPT; ++i) {
        tq[i] = ((const T*)&qreg[i])[e];
        tg[i] = ((const T*)&greg[i])[e];
      }
      store_bytes<C::QKPT * (int)sizeof(T)>(QT + (sc * C::E + e) * C::QTs + sg * C::QKPT, tq);
      store_bytes<C::QKPT * (int)sizeof(T)>(OT + (sc * C::E + e) * C::QTs + sg * C::QKPT, tg);
    }
    if (tid < BR) {
      LS[tid] = lreg;
      DD[tid] = dreg;
    }
  };

  f32x16 dk[C::DBLK], dv[C::DBLK];
#pragma unroll
  for (int i = 0; i < C::DBLK; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  const float c = a.c;
  const int prow = acc_row_to_key(l32);

  if (qt_begin < n_qt) {
    gload(qt_begin);
    lstore();
  }
  __syncthreads();

  for (int qt = qt_begin; qt < n_qt; ++qt) {
    const int q0 = qt * BR;
    const bool more = qt + 1 < n_qt;
    if (more) gload(qt + 1);
    // Waves whose keys all follow the tile's last row see only masked entries.
    const bool active = !CAUSAL || kw0 <= q0 + BR - 1;
    const bool need_mask = (kw0 + 31 >= N) || (CAUSAL && kw0 + 31 > q0);
    if (active) {
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < C::KSTEPS; ++kk) {
          const int col = kk * 2 * KPL + hh * KPL;
          const Frag qa = Tr::load(QS + (qb * 32 + prow) * C::QSs + col);
          s = Tr::mma(qa, kf[kk], s);
          const Frag ga = Tr::load(OS + (qb * 32 + prow) * C::QSs + col);
          dp = Tr::mma(ga, vf[kk], dp);
        }
        // P = exp2(S * c - L * log2 e) and dS = P * (dP - D) at rows q, key = this lane's.
        float p[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qb * 32 + slot_key(r, hh);
          float e = fast_exp2(__builtin_fmaf(s[r], c, -LS[ql]));
          if (need_mask) {
            const bool ok = key_ok && (!CAUSAL || key <= q0 + ql);
            e = ok ? e : 0.f;
          }
          p[r] = e;
          ds[r] = e * (dp[r] - DD[ql]);
        }
        // dV += P^T dO and dK += dS^T Q (scale applied at the end).
#pragma unroll
        for (int ks = 0; ks < C::PSTEPS; ++ks) {
          const Frag pa = Tr::pack(&p[ks * KPL]);
          const Frag da = Tr::pack(&ds[ks * KPL]);
          const int qoff = qb * 32 + slot_key(ks * KPL, hh);
#pragma unroll
          for (int db = 0; db < C::DBLK; ++db) {
            const Frag gb = Tr::load(OT + (db * 32 + l32) * C::QTs + qoff);
            dv[db] = Tr::mma(pa, gb, dv[db]);
            const Frag qbf = Tr::load(QT + (db * 32 + l32) * C::QTs + qoff);
            dk[db] = Tr::mma(da, qbf, dk[db]);
          }
        }
        // dS (rounded like the other operands) to LDS, rows q, columns key.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qb * 32 + slot_key(r, hh);
          DS[ql * C::DSs + wave * 32 + l32] = (T)ds[r];
        }
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) DS[(qb * 32 + slot_key(r, hh)) * C::DSs + wave * 32 + l32] = (T)0.f;
    }
    __syncthreads();
    // Q, dO of this tile are no longer read: stage the next tile while dQ is formed.
    if (more) lstore();
    // dQ[q][d] += sum over the workgroup's keys of dS[q][key] K[key][d], lanes = d.
    for (int bi = wave; bi < C::QB * C::DBLK; bi += 4) {
      const int qb = bi / C::DBLK, db = bi % C::DBLK;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kc = 0; kc < C::CSTEPS; ++kc) {
        const int col = kc * 2 * KPL + hh * KPL;
        const Frag sa = Tr::load(DS + (qb * 32 + l32) * C::DSs + col);
        const Frag kb = Tr::load(KT + (db * 32 + l32) * C::KTs + col);
        acc = Tr::mma(sa, kb, acc);
      }
      const int d = db * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + qb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (q < N) unsafeAtomicAdd(dQg + (size_t)q * D + d, acc[r]);
      }
    }
    __syncthreads();
  }

  // Epilogue: dK = scale * acc, dV = acc; lanes = d, rows = keys.
  T* dKg = (T*)a.dk + base;
  T* dVg = (T*)a.dv + base;
  const float scale = a.scale;
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (kr < N) {
        const size_t off = (size_t)kr * D + db * 32 + l32;
        dKg[off] = (T)(dk[db][r] * scale);
        dVg[off] = (T)dv[db][r];
      }
    }
}

template <class Tr, int D, bool CAUSAL>
hipError_t launch_main(const BwdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((bwd_main_kernel<Tr, D, CAUSAL>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <class Tr, int D>
hipError_t run(int causal, BwdArgs a, int B, int H, int stage_mask, hipStream_t s) {
  using T = typename Tr::T;
  constexpr int E = 16 / sizeof(T);
  const long long rows = (long long)B * H * a.N;
  if (stage_mask & 1) {
    const long long threads = rows * (D / E);
    const int blocks = (int)((threads + kThreads - 1) / kThreads);
    hipLaunchKernelGGL((bwd_pre_kernel<Tr, D>), dim3(blocks), dim3(kThreads), 0, s, a, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage_mask & 2) {
    if constexpr (sizeof(typename Tr::T) == 2) {
      hipError_t e = launch_bwd_bf16_main(D, causal, a, B, H, s);
      if (e != hipSuccess) return e;
    } else {
    a.n_tiles = (a.N + kBC - 1) / kBC;
    const long long grid = (long long)B * H * a.n_tiles;
    a.remap = grid % 8 == 0 ? 1 : 0;
    hipError_t e = causal ? launch_main<Tr, D, true>(a, (int)grid, s) : launch_main<Tr, D, false>(a, (int)grid, s);
    if (e != hipSuccess) return e;
    }
  }
  if (stage_mask & 4) {
    const long long n4 = rows * D / 4;
    const int blocks = (int)((n4 + kThreads - 1) / kThreads);
    hipLaunchKernelGGL((bwd_dq_kernel<Tr, D>), dim3(blocks), dim3(kThreads), 0, s, a, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (sizeof(typename Tr::T) == 2) {
      if (a.dkv_part != nullptr) {   // grouped K/V heads
        const long long m4 = (long long)B * (H / a.group) * a.N * D / 4;
        const int mb = (int)((m4 + kThreads - 1) / kThreads);
        hipLaunchKernelGGL((bwd_dkv_sum_kernel<D>), dim3(mb), dim3(kThreads), 0, s, a, m4);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(DType dt, int d, int causal, BwdArgs a, int B, int H, int stage_mask, hipStream_t s) {
  if (dt == DType::BF16) return d == 64 ? run<TrBF16, 64>(causal, a, B, H, stage_mask, s)
                                        : run<TrBF16, 128>(causal, a, B, H, stage_mask, s);
  return d == 64 ? run<TrF32, 64>(causal, a, B, H, stage_mask, s) : run<TrF32, 128>(causal, a, B, H, stage_mask, s);
}

}  // namespace fa
