// C ABI of the library: argument checks, then one asynchronous launch
// sequence on the caller's stream. See include/fa.h for the contract.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <algorithm>
#include <cstdio>
#include <mutex>

#include "fa.h"
#include "fa_kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return FA_OK;
}

struct Buf {
  const void* p;
  size_t bytes;
  const char* name;
  size_t align;
};

bool overlaps(const Buf& a, const Buf& b) {
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Sizes, head dimension and scale.
int check_shape(int B, int H, int N, int d, float scale) {
  if (B < 1 || H < 1 || N < 1)
    return fail(FA_ERR_INVALID, "B, H and N must be >= 1 (got B=%d H=%d N=%d)", B, H, N);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension d must be 64 or 128 (got %d)", d);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(FA_ERR_UNSUPPORTED, "scale must be finite and >= 0 (got %g)", (double)scale);
  // Kernels address one (batch, head) with 32-bit byte offsets.
  if ((long long)N * d * 4 > (1LL << 30))
    return fail(FA_ERR_UNSUPPORTED, "sequence too long: N * d = %lld exceeds 2^28 elements per head",
                (long long)N * d);
  const long long tiles = (long long)B * H * ((N + 63) / 64);
  if (tiles > INT_MAX / 2 || (long long)B * H * N > INT_MAX)
    return fail(FA_ERR_UNSUPPORTED, "problem too large: B*H*N = %lld exceeds the supported range",
                (long long)B * H * N);
  return FA_OK;
}

// Null, alignment and overlap checks. inputs/outputs are arrays of n buffers.
int check_bufs(const Buf* in, int n_in, const Buf* out, int n_out) {
  for (int i = 0; i < n_in + n_out; ++i) {
    const Buf& b = i < n_in ? in[i] : out[i - n_in];
    if (b.p == nullptr) return fail(FA_ERR_INVALID, "%s is NULL", b.name);
    if ((uintptr_t)b.p % b.align != 0)
      return fail(FA_ERR_UNSUPPORTED, "%s must be %zu-byte aligned", b.name, b.align);
  }
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(out[i], in[j]))
        return fail(FA_ERR_INVALID, "output %s overlaps input %s", out[i].name, in[j].name);
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(out[i], out[j]))
        return fail(FA_ERR_INVALID, "outputs %s and %s overlap", out[i].name, out[j].name);
  }
  return FA_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

float log2e_scale(float scale) { return (float)((double)scale * 1.4426950408889634); }

// K/V heads: 1 <= H_kv <= H with H a multiple of H_kv.
int check_kv_heads(int H, int H_kv) {
  if (H_kv < 1 || H_kv > H || H % H_kv != 0)
    return fail(FA_ERR_INVALID, "H = %d query heads must be a multiple of H_kv = %d >= 1 K/V heads", H, H_kv);
  return FA_OK;
}

int fwd_common(fa::DType dt, const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, void* stream, int H_kv = 0) {
  if (H_kv == 0) H_kv = H;   // (callers without grouped heads)
  int rc = check_shape(B, H, N, d, scale);
  if (rc) return rc;
  rc = check_kv_heads(H, H_kv);
  if (rc) return rc;
  const size_t e = dt == fa::DType::BF16 ? 2 : 4;
  const size_t tb = (size_t)B * H * N * d * e, kb = (size_t)B * H_kv * N * d * e, lb = (size_t)B * H * N * 4;
  const Buf in[3] = {{q, tb, "q", 16}, {k, kb, "k", 16}, {v, kb, "v", 16}};
  const Buf out[2] = {{o, tb, "o", 16}, {lse, lb, "lse", 4}};
  rc = check_bufs(in, 3, out, 2);
  if (rc) return rc;
  fa::FwdArgs a{q, k, v, o, lse, N, 0, log2e_scale(scale), 0, H, H / H_kv};
  return launched(fa::launch_fwd(dt, d, causal, a, B, H, (hipStream_t)stream), "attention forward");
}

int bwd_common(fa::DType dt, const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, int B, int H, int N,
               int d, float scale, int causal, void* stream, int stage_mask = 7, bool det = false, int H_kv = 0) {
  if (H_kv == 0) H_kv = H;   // (callers without grouped heads)
  if (stage_mask < 1 || stage_mask > 7) return fail(FA_ERR_INVALID, "stage_mask must be in 1..7 (got %d)", stage_mask);
  int rc = check_shape(B, H, N, d, scale);
  if (rc) return rc;
  rc = check_kv_heads(H, H_kv);
  if (rc) return rc;
  const size_t need = det ? fa_bwd_det_workspace_bytes(B, H, N, d, causal)
                     : H_kv < H ? fa_bwd_gqa_workspace_bytes(B, H, H_kv, N, d) : fa_bwd_workspace_bytes(B, H, N, d);
  if (ws == nullptr) return fail(FA_ERR_INVALID, "workspace is NULL");
  if ((uintptr_t)ws % 256 != 0) return fail(FA_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(FA_ERR_INVALID, "workspace has %zu bytes, needs %s() = %zu", ws_bytes,
                det ? "fa_bwd_det_workspace_bytes" : H_kv < H ? "fa_bwd_gqa_workspace_bytes" : "fa_bwd_workspace_bytes",
                need);
  const size_t e = dt == fa::DType::BF16 ? 2 : 4;
  const size_t tb = (size_t)B * H * N * d * e, kb = (size_t)B * H_kv * N * d * e, lb = (size_t)B * H * N * 4;
  const Buf in[6] = {{q, tb, "q", 16},   {k, kb, "k", 16},     {v, kb, "v", 16},
                     {o, tb, "o", 16},   {lse, lb, "lse", 4},  {dout, tb, "dout", 16}};
  const Buf out[4] = {{dq, tb, "dq", 16}, {dk, kb, "dk", 16}, {dv, kb, "dv", 16}, {ws, need, "workspace", 256}};
  rc = check_bufs(in, 6, out, 4);
  if (rc) return rc;
  fa::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.N = N; a.scale = scale; a.c = log2e_scale(scale);
  a.H = H; a.group = H / H_kv; a.B = B;
  a.dq_acc = (float*)ws;
  a.dvec = (float*)((char*)ws + align256((size_t)B * H * N * d * 4));
  if (det) {
    // fixed order: the per-query-tile counters and the error flag after D
    const size_t n_cnt = (size_t)B * H * fa::bwd_row_tiles(N) * fa::kBwdSlots;
    a.dq_cnt = (int*)((char*)ws + fa_bwd_workspace_bytes(B, H, N, d));
    a.dq_err = a.dq_cnt + n_cnt;
    a.n_cnt = (int)(n_cnt + 1);
  } else if (H_kv < H) {
    // grouped K/V heads: float32 dK, dV per query head after D
    a.dkv_part = (float*)((char*)ws + fa_bwd_workspace_bytes(B, H, N, d));
  }
  return launched(fa::launch_bwd(dt, d, causal, a, B, H, stage_mask, (hipStream_t)stream), "attention backward");
}

// ---- scratch of the allocation-free backward (fa_bwd_noalloc).
//
// One fixed array per device, resident while the library is loaded. In host
// code the name `scratch` stands for the host-side shadow, not for the
// device memory: the device address comes from hipGetSymbolAddress, looked
// up once per device with that device current, and only that address is
// ever passed to kernels.
constexpr size_t kScratchBytes = (size_t)128 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// *out = device address of this device's scratch array; a non-OK status
// (with the error text set) if it cannot be found.
int scratch_on_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char*)g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported argument";
    case FA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* fa_last_error(void) { return g_err; }

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, void* stream) {
  return fwd_common(fa::DType::BF16, q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
  return fwd_common(fa::DType::F32, q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return align256((size_t)B * H * N * d * 4) + align256((size_t)B * H * N * 4);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
           float scale, int causal, void* stream) {
  return bwd_common(fa::DType::BF16, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                    scale, causal, stream);
}

int fa_bwd_stages(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                  float scale, int causal, int stage_mask, void* stream) {
  return bwd_common(fa::DType::BF16, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                    scale, causal, stream, stage_mask);
}

size_t fa_bwd_det_workspace_bytes(int B, int H, int N, int d, int causal) {
  (void)causal;   // the same for both masks
  const size_t base = fa_bwd_workspace_bytes(B, H, N, d);
  if (base == 0) return 0;
  // counters: kBwdSlots per (batch, head, 32-row query tile), then the error flag
  return base + align256(((size_t)B * H * fa::bwd_row_tiles(N) * fa::kBwdSlots + 1) * 4);
}

int fa_bwd_det(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
  return bwd_common(fa::DType::BF16, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                    scale, causal, stream, 7, true);
}

size_t fa_bwd_gqa_workspace_bytes(int B, int H, int H_kv, int N, int d) {
  const size_t base = fa_bwd_workspace_bytes(B, H, N, d);
  if (base == 0 || H_kv < 1 || H_kv > H || H % H_kv != 0) return 0;
  // grouped K/V heads: float32 dK and dV per query head, [B H_kv][G][N][d] each
  return H_kv < H ? base + align256((size_t)2 * B * H * N * d * 4) : base;
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N,
               int d, float scale, int causal, void* stream) {
  if (H_kv < 1) return check_kv_heads(H, H_kv);
  return fwd_common(fa::DType::BF16, q, k, v, o, lse, B, H, N, d, scale, causal, stream, H_kv);
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int H_kv,
               int N, int d, float scale, int causal, void* stream) {
  if (H_kv < 1) return check_kv_heads(H, H_kv);
  return bwd_common(fa::DType::BF16, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                    scale, causal, stream, 7, false, H_kv);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens,
                  int n_seq, int max_seqlen, int total, int H, int H_kv, int d, float scale, int causal,
                  void* stream) {
  int rc = check_shape(1, H, total, d, scale);
  if (rc) return rc;
  if (H_kv < 1) return check_kv_heads(H, H_kv);
  rc = check_kv_heads(H, H_kv);
  if (rc) return rc;
  if (n_seq < 1 || max_seqlen < 1 || max_seqlen > total)
    return fail(FA_ERR_INVALID, "need n_seq >= 1 and 1 <= max_seqlen <= total (got n_seq=%d max_seqlen=%d total=%d)",
                n_seq, max_seqlen, total);
  if ((long long)n_seq * H * ((max_seqlen + 255) / 256) > INT_MAX / 2)
    return fail(FA_ERR_UNSUPPORTED, "too many sequences: n_seq = %d", n_seq);
  const size_t tb = (size_t)H * total * d * 2, kb = (size_t)H_kv * total * d * 2, lb = (size_t)H * total * 4;
  const Buf in[4] = {{q, tb, "q", 16}, {k, kb, "k", 16}, {v, kb, "v", 16},
                     {cu_seqlens, (size_t)(n_seq + 1) * 4, "cu_seqlens", 4}};
  const Buf out[2] = {{o, tb, "o", 16}, {lse, lb, "lse", 4}};
  rc = check_bufs(in, 4, out, 2);
  if (rc) return rc;
  fa::FwdArgs a{q, k, v, o, lse, total, 0, log2e_scale(scale), 0, H, H / H_kv, cu_seqlens, max_seqlen};
  return launched(fa::launch_fwd(fa::DType::BF16, d, causal, a, n_seq, H, (hipStream_t)stream),
                  "variable-length attention forward");
}

size_t fa_bwd_varlen_workspace_bytes(int total, int H, int H_kv, int d) {
  const size_t base = fa_bwd_workspace_bytes(1, H, total, d);
  if (base == 0 || H_kv < 1 || H_kv > H || H % H_kv != 0) return 0;
  // grouped heads: float32 dK, dV per query head, [H_kv][G][total][d] each
  return H_kv < H ? base + align256((size_t)2 * H * total * d * 4) : base;
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, const int* cu_seqlens,
                  int n_seq, int max_seqlen, int total, int H, int H_kv, int d, float scale, int causal,
                  void* stream) {
  int rc = check_shape(1, H, total, d, scale);
  if (rc) return rc;
  if (H_kv < 1) return check_kv_heads(H, H_kv);
  rc = check_kv_heads(H, H_kv);
  if (rc) return rc;
  if (n_seq < 1 || max_seqlen < 1 || max_seqlen > total)
    return fail(FA_ERR_INVALID, "need n_seq >= 1 and 1 <= max_seqlen <= total (got n_seq=%d max_seqlen=%d total=%d)",
                n_seq, max_seqlen, total);
  if ((long long)n_seq * H * ((max_seqlen + 255) / 256) > INT_MAX / 2)
    return fail(FA_ERR_UNSUPPORTED, "too many sequences: n_seq = %d", n_seq);
  const size_t need = fa_bwd_varlen_workspace_bytes(total, H, H_kv, d);
  if (workspace == nullptr) return fail(FA_ERR_INVALID, "workspace is NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(FA_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID, "workspace has %zu bytes, needs fa_bwd_varlen_workspace_bytes() = %zu",
                workspace_bytes, need);
  const size_t tb = (size_t)H * total * d * 2, kb = (size_t)H_kv * total * d * 2, lb = (size_t)H * total * 4;
  const Buf in[7] = {{q, tb, "q", 16},   {k, kb, "k", 16},    {v, kb, "v", 16},
                     {o, tb, "o", 16},   {lse, lb, "lse", 4}, {dout, tb, "dout", 16},
                     {cu_seqlens, (size_t)(n_seq + 1) * 4, "cu_seqlens", 4}};
  const Buf out[4] = {{dq, tb, "dq", 16}, {dk, kb, "dk", 16}, {dv, kb, "dv", 16}, {workspace, need, "workspace", 256}};
  rc = check_bufs(in, 7, out, 4);
  if (rc) return rc;
  fa::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.N = total; a.scale = scale; a.c = log2e_scale(scale);
  a.H = H; a.group = H / H_kv; a.B = 1;
  a.cu_seqlens = cu_seqlens; a.n_seq = n_seq; a.max_seqlen = max_seqlen;
  a.dq_acc = (float*)workspace;
  a.dvec = (float*)((char*)workspace + align256((size_t)H * total * d * 4));
  if (H_kv < H) a.dkv_part = (float*)((char*)workspace + fa_bwd_workspace_bytes(1, H, total, d));
  return launched(fa::launch_bwd(fa::DType::BF16, d, causal, a, 1, H, 7, (hipStream_t)stream),
                  "variable-length attention backward");
}

size_t fa_bwd_noalloc_scratch_bytes(void) { return kScratchBytes; }

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                   void* stream) {
  int rc = check_shape(B, H, N, d, scale);
  if (rc) return rc;
  const size_t tb = (size_t)B * H * N * d * 2, lb = (size_t)B * H * N * 4;
  const Buf in[6] = {{q, tb, "q", 16},   {k, tb, "k", 16},     {v, tb, "v", 16},
                     {o, tb, "o", 16},   {lse, lb, "lse", 4},  {dout, tb, "dout", 16}};
  const Buf out[3] = {{dq, tb, "dq", 16}, {dk, tb, "dk", 16}, {dv, tb, "dv", 16}};
  rc = check_bufs(in, 6, out, 3);
  if (rc) return rc;
  // Heads are independent and contiguous, so they run in chunks whose
  // workspace fits the scratch array, one after another on the stream.
  const size_t per_head = fa_bwd_workspace_bytes(1, 1, N, d);
  if (per_head > kScratchBytes)
    return fail(FA_ERR_UNSUPPORTED,
                "fa_bwd_noalloc: one head of N = %d, d = %d needs %zu bytes of workspace; the scratch holds %zu",
                N, d, per_head, kScratchBytes);
  const int heads = B * H;
  int chunk = (int)std::min<size_t>((size_t)heads, kScratchBytes / per_head);
  while (chunk > 1 && fa_bwd_workspace_bytes(1, chunk, N, d) > kScratchBytes) --chunk;
  char* ws = nullptr;
  rc = scratch_on_current_device(&ws);
  if (rc) return rc;
  const size_t head_elems = (size_t)N * d;
  for (int h0 = 0; h0 < heads; h0 += chunk) {
    const int c = std::min(chunk, heads - h0);
    fa::BwdArgs a{};
    const size_t eo = (size_t)h0 * head_elems * 2;   // bytes into the bf16 tensors
    a.q = (const char*)q + eo; a.k = (const char*)k + eo; a.v = (const char*)v + eo;
    a.o = (const char*)o + eo; a.lse = lse + (size_t)h0 * N; a.dout = (const char*)dout + eo;
    a.dq = (char*)dq + eo; a.dk = (char*)dk + eo; a.dv = (char*)dv + eo;
    a.N = N; a.scale = scale; a.c = log2e_scale(scale);
    a.H = c; a.group = 1; a.B = 1;
    a.dq_acc = (float*)ws;
    a.dvec = (float*)(ws + align256((size_t)c * N * d * 4));
    rc = launched(fa::launch_bwd(fa::DType::BF16, d, causal, a, 1, c, 7, (hipStream_t)stream),
                  "attention backward (no allocation)");
    if (rc) return rc;
  }
  return ok();
}

int fa_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse,
               const float* dout, float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes, int B,
               int H, int N, int d, float scale, int causal, void* stream) {
  return bwd_common(fa::DType::F32, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                    scale, causal, stream);
}

int fa_quant_fp8(const void* x, const float* rot, unsigned char* x8, float* scales, int B, int H, int N, int d,
                 int block_rows, int pow2, void* stream) {
  int rc = check_shape(B, H, N, d, 1.f);
  if (rc) return rc;
  if (block_rows != 64 && block_rows != 0)
    return fail(FA_ERR_UNSUPPORTED, "block_rows must be 64 or 0 (got %d)", block_rows);
  if (pow2 != 0 && pow2 != 1) return fail(FA_ERR_INVALID, "pow2 must be 0 or 1 (got %d)", pow2);
  const size_t n = (size_t)B * H * N * d;
  const size_t sb = (size_t)B * H * ((N + 63) / 64) * 4;
  const Buf in_r[2] = {{x, n * 2, "x", 16}, {rot, (size_t)d * d * 4, "rot", 16}};
  const Buf out[2] = {{x8, n, "x8", 16}, {scales, sb, "scales", 4}};
  rc = check_bufs(in_r, rot ? 2 : 1, out, 2);
  if (rc) return rc;
  fa::QuantArgs a{x, rot, x8, scales, N, block_rows, pow2};
  return launched(fa::launch_quant_fp8(d, a, B, H, (hipStream_t)stream), "fp8 quantisation");
}

int fa_dequant_fp8(const unsigned char* x8, const float* scales, int block_rows, void* out, int B, int H, int N,
                   int d, void* stream) {
  int rc = check_shape(B, H, N, d, 1.f);
  if (rc) return rc;
  if (block_rows != 64 && block_rows != 0)
    return fail(FA_ERR_UNSUPPORTED, "block_rows must be 64 or 0 (got %d)", block_rows);
  const size_t n = (size_t)B * H * N * d;
  const size_t sb = (size_t)B * H * ((N + 63) / 64) * 4;
  const Buf in[2] = {{x8, n, "x8", 16}, {scales, sb, "scales", 4}};
  const Buf out_[1] = {{out, n * 2, "out", 16}};
  rc = check_bufs(in, 2, out_, 1);
  if (rc) return rc;
  return launched(fa::launch_dequant_fp8(x8, scales, out, B, H, N, d, (hipStream_t)stream), "fp8 decoding");
}

size_t fa_bwd_fp8_workspace_bytes(int B, int H, int N, int d) {
  const size_t base = fa_bwd_workspace_bytes(B, H, N, d);
  if (base == 0) return 0;
  // the bf16 backward's workspace, then the decoded Q, K and V (bf16)
  return base + 3 * align256((size_t)B * H * N * d * 2);
}

int fa_bwd_fp8(const unsigned char* q8, const unsigned char* k8, const unsigned char* v8, const float* sq,
               const float* sk, const float* sv, int block_rows, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
  int rc = check_shape(B, H, N, d, scale);
  if (rc) return rc;
  if (block_rows != 64 && block_rows != 0)
    return fail(FA_ERR_UNSUPPORTED, "block_rows must be 64 or 0 (got %d)", block_rows);
  const size_t need = fa_bwd_fp8_workspace_bytes(B, H, N, d);
  if (workspace == nullptr) return fail(FA_ERR_INVALID, "workspace is NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(FA_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID, "workspace has %zu bytes, needs fa_bwd_fp8_workspace_bytes() = %zu",
                workspace_bytes, need);
  const size_t n = (size_t)B * H * N * d;
  const size_t sb = (size_t)B * H * ((N + 63) / 64) * 4;
  const size_t lb = (size_t)B * H * N * 4;
  const Buf in[9] = {{q8, n, "q8", 16},  {k8, n, "k8", 16},   {v8, n, "v8", 16},
                     {sq, sb, "sq", 4},  {sk, sb, "sk", 4},   {sv, sb, "sv", 4},
                     {o, n * 2, "o", 16}, {lse, lb, "lse", 4}, {dout, n * 2, "dout", 16}};
  const Buf out[4] = {{dq, n * 2, "dq", 16}, {dk, n * 2, "dk", 16}, {dv, n * 2, "dv", 16},
                      {workspace, need, "workspace", 256}};
  rc = check_bufs(in, 9, out, 4);
  if (rc) return rc;
  // Decoded Q, K, V after the bf16 backward's own workspace.
  const size_t base = fa_bwd_workspace_bytes(B, H, N, d);
  const size_t tb = align256(n * 2);
  char* dec = (char*)workspace + base;
  const hipStream_t st = (hipStream_t)stream;
  const unsigned char* codes[3] = {q8, k8, v8};
  const float* scales[3] = {sq, sk, sv};
  for (int t = 0; t < 3; ++t) {
    rc = launched(fa::launch_dequant_fp8(codes[t], scales[t], dec + t * tb, B, H, N, d, st), "fp8 decoding");
    if (rc) return rc;
  }
  return bwd_common(fa::DType::BF16, dec, dec + tb, dec + 2 * tb, o, lse, dout, dq, dk, dv, workspace, base, B, H,
                    N, d, scale, causal, stream);
}

int fa_fwd_fp8(const unsigned char* q8, const unsigned char* k8, const unsigned char* v8, const float* sq,
               const float* sk, const float* sv, int block_rows, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
  int rc = check_shape(B, H, N, d, scale);
  if (rc) return rc;
  // Both granularities fa_quant_fp8 writes share one layout (a per-tensor
  // scale is broadcast to every 64-row entry), so the kernel reads them alike.
  if (block_rows != 64 && block_rows != 0)
    return fail(FA_ERR_UNSUPPORTED, "block_rows must be 64 or 0 (got %d)", block_rows);
  if (d != 128) return fail(FA_ERR_UNSUPPORTED, "fp8 forward supports d = 128 only (got %d)", d);
  const size_t n = (size_t)B * H * N * d;
  const size_t sb = (size_t)B * H * ((N + 63) / 64) * 4;
  const Buf in[6] = {{q8, n, "q8", 16}, {k8, n, "k8", 16}, {v8, n, "v8", 16},
                     {sq, sb, "sq", 4},  {sk, sb, "sk", 4},  {sv, sb, "sv", 4}};
  const Buf out[2] = {{o, n * 2, "o", 16}, {lse, (size_t)B * H * N * 4, "lse", 4}};
  rc = check_bufs(in, 6, out, 2);
  if (rc) return rc;
  fa::Fp8FwdArgs a{q8, k8, v8, sq, sk, sv, o, lse, N, 0, log2e_scale(scale), 0};
  return launched(fa::launch_fwd_fp8(d, causal, a, B, H, (hipStream_t)stream), "fp8 attention forward");
}

}  // extern "C"
