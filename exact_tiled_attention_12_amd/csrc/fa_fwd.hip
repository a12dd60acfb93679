// Fused exact-attention forward for gfx950: float32 inputs (this file) and the
// bf16 entry (fa_fwd_bf16.hip).
//
// What it computes ("FlashAttention v1～v4 完整进化史", v1 pseudocode and v2
// part 1; "6.1 FlashAttention V1详解", section 5.1): for one query tile the
// workgroup keeps the running row maximum m, the rescaled exponent sum l and
// an unnormalised output accumulator, walks the key/value tiles once, and
// writes O = acc / l and L = m + log l at the end. The score and probability
// tiles live only in registers.
//
// MI355X mapping:
//   * one workgroup (4 waves, 256 threads) per (batch, head, 128-row query
//     tile); each wave owns 32 query rows (the v2 split of query rows over
//     warps, "FlashAttention v1～v4 完整进化史" v2 part 3, on wave64);
//   * key/value tiles of 64 rows are staged in LDS, double buffered: the
//     global loads of tile j+1 are issued before tile j is computed and
//     written to the other buffer afterwards;
//   * the kernel forms S^T = K Q^T and O^T = V^T P^T on the 32x32 MFMA, with
//     the rows of K permuted (acc_row_to_key) so that every lane owns one
//     query and its 8-key runs of exp'd scores are directly the operand of
//     the second product: P never leaves registers;
//   * V is transposed while it is written to LDS so each lane reads its
//     8-key operand run with one 16-byte LDS read;
//   * the row max/sum need one exchange between the two lane halves
//     (v_permlane32_swap); exp goes through v_exp_f32 (base 2) with
//     scale * log2(e) folded into one FMA per score;
//   * causal grids issue the heaviest query tiles first; ids are remapped so
//     the tiles of one (batch, head) share an XCD (and its L2).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kBR = 128;   // query rows per workgroup
constexpr int kBC = 64;    // keys per tile
constexpr int kThreads = 256;

template <class Tr, int D>
struct FwdCfg {
  using T = typename Tr::T;
  static constexpr int E = 16 / sizeof(T);            // elements per 16-byte chunk
  static constexpr int KS = D + E;                    // LDS row stride of K (elements)
  static constexpr int VS = kBC + E;                  // LDS row stride of V^T (elements)
  static constexpr int K_ELEMS = kBC * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;       // one stage
  static constexpr int CPR = D / E;                   // 16-byte chunks per row
  static constexpr int K_PER_T = kBC * CPR / kThreads;
  static constexpr int VG = kThreads / CPR;           // key groups for the V transpose
  static constexpr int KPT = kBC / VG;                // keys per thread in the V transpose
  static constexpr int KSTEPS = D / (2 * Tr::KPL);    // MFMA steps over d
  static constexpr int PSTEPS = 32 / (2 * Tr::KPL);   // MFMA steps over 32 keys
  static constexpr int DBLK = D / 32;
  static constexpr int LDS_BYTES = 2 * BUF * (int)sizeof(T);
  static_assert(K_PER_T * kThreads == kBC * CPR, "K tile split");
  static_assert(KPT * VG == kBC, "V tile split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class Tr, int D, bool CAUSAL, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void fwd_kernel(FwdArgs a) {
  using C = FwdCfg<Tr, D>;
  using T = typename Tr::T;
  using Frag = typename Tr::Frag;
  constexpr int KPL = Tr::KPL;
  __shared__ __attribute__((aligned(16))) T lds[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  int wg = blockIdx.x;
  if (a.remap) wg = xcd_remap(wg, gridDim.x);
  const int bh = wg / a.n_qtiles;
  const int t = wg - bh * a.n_qtiles;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - t) : t;
  const int N = a.N;
  const size_t base = (size_t)bh * (size_t)N * D;
  const T* __restrict__ Qg = (const T*)a.q + base;
  const T* __restrict__ Kg = (const T*)a.k + base;
  const T* __restrict__ Vg = (const T*)a.v + base;
  T* __restrict__ Og = (T*)a.o + base;

  const int q0 = qt * kBR;
  const int wrow0 = q0 + wave * 32;
  const int qrow = wrow0 + l32;

  // Q rows of this wave as the B operand of S^T = K Q^T (read once).
  Frag qf[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk)
    qf[kk] = qrow < N ? Tr::load(Qg + (size_t)qrow * D + kk * 2 * KPL + hh * KPL) : Tr::zero();

  const int n_kv = (N + kBC - 1) / kBC;
  int kv_end = n_kv;
  if (CAUSAL) kv_end = min(n_kv, (min(q0 + kBR, N) - 1) / kBC + 1);

  // Global -> register stage of one key/value tile.
  u32x4 kreg[C::K_PER_T];
  u32x4 vreg[C::KPT];
  const int vc = tid % C::CPR, vg = tid / C::CPR;
  auto gload = [&](int j) {
    const int key0 = j * kBC;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / C::CPR, col = c % C::CPR;
      const int g = key0 + row;
      kreg[i] = g < N ? *(const u32x4*)(Kg + (size_t)g * D + col * C::E) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < C::KPT; ++r) {
      const int g = key0 + vg * C::KPT + r;
      vreg[r] = g < N ? *(const u32x4*)(Vg + (size_t)g * D + vc * C::E) : u32x4{0, 0, 0, 0};
    }
  };
  // Register -> LDS: K row-major, V transposed (V^T[d][key]).
  auto lstore = [&](int buf) {
    T* Ks = lds + buf * C::BUF;
    T* Vt = Ks + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / C::CPR, col = c % C::CPR;
      *(u32x4*)(Ks + row * C::KS + col * C::E) = kreg[i];
    }
#pragma unroll
    for (int e = 0; e < C::E; ++e) {
      T tmp[C::KPT];
#pragma unroll
      for (int r = 0; r < C::KPT; ++r) tmp[r] = ((const T*)&vreg[r])[e];
      store_bytes<C::KPT * (int)sizeof(T)>(Vt + (vc * C::E + e) * C::VS + vg * C::KPT, tmp);
    }
  };

  const float c = a.c;
  float m = -INFINITY;      // running max of scale*log2(e)*s (this lane's row)
  float l = 0.f;            // running sum over this lane half's keys
  f32x16 oacc[C::DBLK];
#pragma unroll
  for (int i = 0; i < C::DBLK; ++i) oacc[i] = f32x16{};
  const int prow = acc_row_to_key(l32);

  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < kv_end; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < kv_end;
    if (more) gload(j + 1);
    const int key0 = j * kBC;
    // A wave whose rows all precede the tile's first key has nothing to do.
    const bool active = !CAUSAL || key0 <= wrow0 + 31;
    if (active) {
      const T* Ks = lds + buf * C::BUF;
      const T* Vt = Ks + C::K_ELEMS;
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int kk = 0; kk < C::KSTEPS; ++kk) {
          const Frag af = Tr::load(Ks + (kb * 32 + prow) * C::KS + kk * 2 * KPL + hh * KPL);
          s[kb] = Tr::mma(af, qf[kk], s[kb]);
        }
      }
      const bool need_mask = (key0 + kBC > N) || (CAUSAL && key0 + kBC - 1 > wrow0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + slot_key(r, hh);
            const bool ok = key < N && (!CAUSAL || key <= qrow);
            s[kb][r] = ok ? s[kb][r] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = halves_max(mx);
      const float mxs = mx == -INFINITY ? -INFINITY : mx * c;
      const float m_new = fmaxf(m, mxs);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float p[32];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_use));
          if (need_mask) e = s[kb][r] == -INFINITY ? 0.f : e;
          p[kb * 16 + r] = e;
          rs += e;
        }
      l = l * alpha + rs;
      m = m_new;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) oacc[db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < C::PSTEPS; ++ks) {
          const Frag pb = Tr::pack(&p[kb * 16 + ks * KPL]);
          const int koff = kb * 32 + slot_key(ks * KPL, hh);
#pragma unroll
          for (int db = 0; db < C::DBLK; ++db) {
            const Frag va = Tr::load(Vt + (db * 32 + l32) * C::VS + koff);
            oacc[db] = Tr::mma(va, pb, oacc[db]);
          }
        }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

  const float lt = halves_sum(l);
  if (qrow < N) {
    // l = 0 only for a row that saw no key (O = 0, LSE = -inf); NaN propagates.
    const float inv = lt == 0.f ? 0.f : 1.f / lt;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hh;
        T* dst = Og + (size_t)qrow * D + d0;
        if constexpr (sizeof(T) == 2) {
          u32x2 w;
          w[0] = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
          w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
          *(u32x2*)dst = w;
        } else {
          f32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = oacc[db][4 * g + i] * inv;
          *(f32x4*)dst = w;
        }
      }
    if (hh == 0)
      a.lse[(size_t)bh * N + qrow] = lt == 0.f ? -INFINITY : (m + fast_log2(lt)) * kLn2;
  }
}

template <class Tr, int D, bool CAUSAL, int OCC>
hipError_t launch_one(const FwdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((fwd_kernel<Tr, D, CAUSAL, OCC>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <class Tr, int OCC>
hipError_t dispatch(int d, int causal, const FwdArgs& a, int grid, hipStream_t s) {
  if (d == 64) return causal ? launch_one<Tr, 64, true, OCC>(a, grid, s) : launch_one<Tr, 64, false, OCC>(a, grid, s);
  return causal ? launch_one<Tr, 128, true, OCC>(a, grid, s) : launch_one<Tr, 128, false, OCC>(a, grid, s);
}

}  // namespace

hipError_t launch_fwd(DType dt, int d, int causal, FwdArgs a, int B, int H, hipStream_t s) {
  if (dt == DType::BF16) return launch_fwd_bf16(d, causal, a, B, H, s);
  a.n_qtiles = (a.N + kBR - 1) / kBR;
  const long long grid = (long long)B * H * a.n_qtiles;
  a.remap = (grid % 8 == 0) ? 1 : 0;
  return dispatch<TrF32, 1>(d, causal, a, (int)grid, s);
}

}  // namespace fa
