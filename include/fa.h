/*
 * fa.h - C ABI of the MI355X (gfx950) fused exact-attention library.
 *
 * The library computes O = softmax(scale * Q K^T) V one (batch, head, query
 * tile) per workgroup with the online softmax, so that the N x N score and
 * probability matrices never reach device memory, and it saves one
 * log-sum-exp per row for the recompute-based backward.
 *
 * What the calls compute follows these pages:
 *   - "FlashAttention v1～v4 完整进化史" (qscqesze), section "第一层地基":
 *     S = Q K^T / sqrt(d), P = softmax(S), O = P V;
 *   - "6.1 FlashAttention V1详解" (AIInfraGuide), section 8.1: tensors are
 *     [B, H, N, D] and the per-row statistics are [B, H, N];
 *   - "FlashAttention v1～v4 完整进化史", v2 part 1: the saved statistic is
 *     L = m + log(l);
 *   - "6.1 FlashAttention V1详解", sections 6.1-6.2: the backward recomputes
 *     S and P from Q, K and the saved statistic instead of storing them;
 *   - "FlashAttention v1～v4 完整进化史", v3 part 3: fp8 with a scale per
 *     block and Q, K rotated by one random orthogonal matrix.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers on the current HIP device. The
 *     caller owns every buffer; the library never allocates, frees or
 *     synchronises, and keeps no state apart from a thread-local error text.
 *   - Layout: contiguous row-major [B, H, N, d] for Q, K, V, O and the
 *     gradients; [B, H, N] float32 for LSE. B and H are batch dimensions.
 *   - d must be 64 or 128. B, H, N >= 1 with N * d <= 2^28 (one head is
 *     addressed with 32-bit offsets) and B * H * N <= 2^31 - 1. scale must
 *     be finite and >= 0 (the workloads use 1/sqrt(d)).
 *   - causal != 0 applies the lower-triangular mask: query i sees keys
 *     j <= i (the diagonal is kept). N queries and N keys.
 *   - LSE is the natural log of sum_j exp(scale * q_i . k_j) over the keys
 *     query i sees.
 *   - Tensor pointers must be 16-byte aligned; LSE and scale arrays 4-byte.
 *   - Outputs must not overlap inputs. Inputs are only read; outputs are
 *     fully overwritten.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work and returns; results are ready when the
 *     stream reaches them.
 *   - Errors: every argument is checked before anything is enqueued; on a
 *     non-zero return nothing was enqueued (FA_ERR_HIP: a launch failed,
 *     earlier launches of the same call may have been enqueued).
 *     fa_last_error() then describes the failure.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point is exported from the shared library (which is built with
 * hidden default visibility). */
#define FA_API __attribute__((visibility("default")))

enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID = -1,     /* null pointer, a size < 1, overlapping buffers, workspace too small */
    FA_ERR_UNSUPPORTED = -2, /* d not 64/128, scale negative or not finite, misaligned pointer, size too large */
    FA_ERR_HIP = -3          /* the HIP runtime reported an error at launch */
};

/* Forward, bf16 inputs and output (bits of bfloat16 in 2-byte elements).
 * Defined by "6.1 FlashAttention V1详解", sections 3.2 and 5.1 (tiles of K
 * and V swept with the online max m and sum l, O rescaled as they change)
 * and "FlashAttention v1～v4 完整进化史", v2 part 1 (O divided by l once at
 * the end; one statistic L = m + log l saved per row).
 * q, k, v: [B,H,N,d] bf16. o: [B,H,N,d] bf16 (written). lse: [B,H,N] float (written).
 * Scores and the output accumulator are float32; P is rounded to bf16
 * (nearest-even) before it multiplies V; O is rounded to bf16 once. */
FA_API int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/* Forward, float32 inputs and output ("6.1 FlashAttention V1详解", sections
 * 3.2 and 5.1; "FlashAttention v1～v4 完整进化史", v2 part 1). Same contract as
 * fa_fwd; every product and sum is in float32 (P is not rounded). */
FA_API int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/* Bytes of device workspace fa_bwd / fa_bwd_f32 need: a float32 dQ
 * accumulator [B,H,N,d] and D = rowsum(dO * O) [B,H,N] float32, each
 * rounded up to 256 bytes. Linear in N (no N x N buffer: the backward's
 * extra memory is O(N), "6.1 FlashAttention V1详解", section 6.3). Returns 0
 * for invalid sizes. */
FA_API size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/* Backward, bf16 ("6.1 FlashAttention V1详解", sections 6.1-6.2: S and P are
 * recomputed from Q, K and the saved statistic, with D = rowsum(dO * O);
 * "FlashAttention v1～v4 完整进化史", v4 part 4: five products per tile, dQ
 * summed across workgroups with atomic adds). Given the forward's inputs
 * q, k, v, its outputs o and lse, and dout = dL/dO, writes dq, dk, dv =
 * dL/dQ, dL/dK, dL/dV (bf16):
 *   D_i = sum_c dO_ic O_ic,  P = exp(scale Q K^T - LSE) (recomputed),
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
 *   dK = scale dS^T Q.
 * workspace: device memory of at least fa_bwd_workspace_bytes(B,H,N,d)
 * bytes, 256-byte aligned; its contents are undefined on entry and exit.
 * dQ is accumulated with float32 atomics, so dq may differ in the last bits
 * between runs; dk and dv are deterministic. */
FA_API int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/* The stages of fa_bwd, for callers that schedule them themselves (and for
 * timing the main stage alone); what they compute is fa_bwd's ("6.1
 * FlashAttention V1详解", sections 6.1-6.2). fa_bwd runs stage_mask 7 =
 * 1 | 2 | 4:
 *   1  preprocess: D = rowsum(dO * O) and a zeroed float32 dQ accumulator,
 *      both in the workspace;
 *   2  main: the recompute of P and the five products; writes dk and dv and
 *      adds into the dQ accumulator;
 *   4  finish: dq = scale * accumulator, cast to bf16.
 * Bits are run in the order 1, 2, 4. Each stage reads what the earlier
 * stages left in the workspace, so stages of one problem must run in order
 * on one stream with the workspace untouched in between. Same arguments and
 * checks as fa_bwd (bf16); stage_mask outside 1..7 gives FA_ERR_INVALID. */
FA_API int fa_bwd_stages(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes,
                         int B, int H, int N, int d, float scale, int causal, int stage_mask, void* stream);

/* Grouped-query and multi-query attention, bf16 ("FlashAttention v1～v4
 * 完整进化史" names GQA and MQA among the attention features a backend may
 * support). q, o, dq, dout: [B,H,N,d]; k, v, dk, dv: [B,H_kv,N,d] with H a
 * multiple of H_kv; lse: [B,H,N]. The H query heads form H_kv groups of
 * G = H / H_kv consecutive heads, and query head h attends with K/V head
 * h / G (MQA: H_kv = 1; H_kv = H is fa_fwd / fa_bwd). dk and dv of a K/V
 * head are the sums over the G query heads that read it: the backward runs
 * one workgroup per (batch, query head, 256-key tile) with the group's K/V
 * head, writes each query head's float32 dK and dV to the workspace, and a
 * final pass adds them in ascending head order; dk and dv are deterministic.
 * The backward's workspace is fa_bwd_gqa_workspace_bytes(B, H, H_kv, N, d).
 * Same conventions, checks and rounding as fa_fwd / fa_bwd; H_kv out of
 * range or not dividing H gives FA_ERR_INVALID. */
FA_API int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int H_kv, int N, int d, float scale, int causal, void* stream);
FA_API int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes,
                      int B, int H, int H_kv, int N, int d, float scale, int causal, void* stream);
/* Bytes of device workspace fa_bwd_gqa needs: fa_bwd_workspace_bytes(B, H,
 * N, d) plus, when H_kv < H, float32 dK and dV per query head (2 x B x H x
 * N x d x 4 bytes, rounded up to 256).
 * Returns 0 for invalid sizes. */
FA_API size_t fa_bwd_gqa_workspace_bytes(int B, int H, int H_kv, int N, int d);

/* Packed variable-length batches, bf16 ("FlashAttention v1～v4 完整进化史",
 * v4 part 4: variable-length sequences, with causal masks, make the work per
 * tile uneven, and heavier tiles are scheduled first). n_seq sequences are
 * packed along the sequence axis: sequence b is rows cu_seqlens[b] ..
 * cu_seqlens[b+1]-1 of every head. q, o: [H, total, d]; k, v: [H_kv, total, d]
 * (H a multiple of H_kv, grouping as in fa_fwd_gqa); lse: [H, total] float32.
 * A query attends only to the keys of its own sequence (causal: those at or
 * before its position in it). cu_seqlens: DEVICE int32 [n_seq + 1],
 * non-decreasing from 0 to total, every length at most max_seqlen; it is read
 * by the kernels only (the library never synchronises), which clamp each
 * sequence to [0, total) and to max_seqlen, so that malformed values give
 * wrong results but no access outside the buffers. Rows of an empty
 * sequence are not written. One workgroup per (sequence, head, 256-row
 * tile of the longest sequence); causal tiles are issued last tile first, and
 * tiles past their sequence's end exit at once. */
FA_API int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int* cu_seqlens, int n_seq, int max_seqlen, int total,
                         int H, int H_kv, int d, float scale, int causal, void* stream);

/* Backward of fa_fwd_varlen: same packed layout and cu_seqlens contract;
 * dout, dq: [H, total, d]; dk, dv: [H_kv, total, d] (for H_kv < H summed over
 * each K/V head's query heads: float32 per query head in the workspace, then
 * added in ascending head order; deterministic). One workgroup per
 * (sequence, query head, 256-key tile of the longest sequence). dQ as in
 * fa_bwd (float32 atomics). Rows of empty sequences get zero gradients.
 * workspace: at least fa_bwd_varlen_workspace_bytes(total, H, H_kv, d) bytes,
 * 256-byte aligned. */
FA_API int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes,
                         const int* cu_seqlens, int n_seq, int max_seqlen, int total,
                         int H, int H_kv, int d, float scale, int causal, void* stream);
/* fa_bwd_workspace_bytes(1, H, total, d), plus 2 x H x total x d x 4 bytes
 * (rounded up to 256) when H_kv < H. Returns 0 for invalid sizes. */
FA_API size_t fa_bwd_varlen_workspace_bytes(int total, int H, int H_kv, int d);

/* Fixed-order (deterministic) backward, bf16 ("FlashAttention v1～v4 完整进化史",
 * v4 part 4: the deterministic backward reduces dQ across workgroups in a
 * fixed order, ordered with semaphores). Same arguments, layouts, checks and
 * mathematics as fa_bwd, but dq is bit-identical from run to run: every
 * 256-key tile adds its float32 dQ contribution to a 32-row query tile only
 * after a counter of that query tile shows that all lower key tiles have
 * added theirs (and for d = 64, key half 0 before key half 1), so every dQ
 * element is summed in ascending key-tile order; the finish pass scales and
 * rounds to bf16 once. dk and dv are bit-identical to fa_bwd's. Extra memory
 * stays O(B H N d) ("6.1 FlashAttention V1详解", section 6.3).
 * A workgroup waits only on workgroups of its own (batch, head) with lower
 * ids, which are dispatched before it. Each wait is bounded (about a
 * second); one that runs out sets an error flag in the workspace and the
 * call then writes NaN to every element of dq (nothing hangs).
 * workspace: device memory of at least
 * fa_bwd_det_workspace_bytes(B,H,N,d,causal) bytes, 256-byte aligned;
 * contents undefined on entry and exit. */
FA_API int fa_bwd_det(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes,
                      int B, int H, int N, int d, float scale, int causal, void* stream);

/* Bytes of device workspace fa_bwd_det needs: fa_bwd_workspace_bytes(B, H,
 * N, d) (the float32 dQ accumulator and D) plus 4 int32 counters per
 * (batch, head, 32-row query tile) and an int32 error flag, rounded up to
 * 256 bytes: linear in N, the same for both masks. Returns 0 for invalid
 * sizes. */
FA_API size_t fa_bwd_det_workspace_bytes(int B, int H, int N, int d, int causal);

/* fa_bwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Same arguments
 * (minus the workspace), checks, layouts and results as fa_bwd (bf16).
 * The workspace is a fixed array inside the library, one per device,
 * fa_bwd_noalloc_scratch_bytes() = 128 MiB, held while the library is
 * loaded. The (batch, head) pairs run in chunks whose fa_bwd workspace
 * fits it, one chunk after another on the stream, so any B and H are
 * accepted; a single head needing more than the array
 * (fa_bwd_workspace_bytes(1, 1, N, d) > 128 MiB, i.e. N above about
 * 260,000 at d = 128) gives FA_ERR_UNSUPPORTED. Every call on a device
 * shares that device's array: calls that may overlap in time on one
 * device (different streams, or threads) race and must be serialised by
 * the caller. The array's first use on a device looks up its address
 * (hipGetSymbolAddress); nothing is allocated or freed. */
FA_API int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv,
                          int B, int H, int N, int d, float scale, int causal, void* stream);
/* Bytes of the scratch array fa_bwd_noalloc uses (per device). */
FA_API size_t fa_bwd_noalloc_scratch_bytes(void);

/* Backward, float32 tensors ("6.1 FlashAttention V1详解", sections 6.1-6.2).
 * Same contract as fa_bwd. */
FA_API int fa_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse,
               const float* dout, float* dq, float* dk, float* dv,
               void* workspace, size_t workspace_bytes,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/* fp8 quantisation ("FlashAttention v1～v4 完整进化史", v3 part 3).
 * x: [B,H,N,d] bf16. rot: d x d float32 row-major orthogonal matrix or NULL;
 * with rot the quantised tensor is x * rot, formed on the bf16 matrix cores
 * with rot split into three bf16 parts (x is exact in bf16) and float32
 * accumulation; its error stays below the float32 FMA-chain bound
 * d 2^-24 / (1 - d 2^-24) (|x| |rot|).
 * block_rows = 64: one scale per 64 rows x d of each (b,h);
 * block_rows = 0: one scale for the whole tensor (the per-tensor baseline).
 * scales: [B,H,ceil(N/64)] float32 (written; with block_rows = 0 every entry
 * holds the same value). The form of the scale is not stated on the page:
 * pow2 = 0 gives s = amax / 448 (a correctly rounded float32 division; the
 * smallest positive float32 where it underflows), which puts the block's
 * largest magnitude on the top code; pow2 = 1 gives the smallest power of
 * two at or above that value, at least 2^-126 (the block-scale form of the
 * fp8 matrix instructions, which fa_fwd_fp8 requires for V); 1 for an
 * all-zero block in both forms. Other pow2 values give FA_ERR_INVALID.
 * x8 = e4m3fn(x / s), rounded to nearest even after saturating to +-448
 * (x8: [B,H,N,d] bytes, written). Inputs are expected finite: a NaN element
 * gets a NaN code (0x7F or 0xFF) and is left out of its block's amax (with
 * rot, every element of its row is NaN after the product and is treated
 * so). block_rows = 0 runs three launches and uses scales as scratch between
 * them (every entry ends up holding the one scale). */
FA_API int fa_quant_fp8(const void* x, const float* rot, unsigned char* x8, float* scales,
                 int B, int H, int N, int d, int block_rows, int pow2, void* stream);

/* Forward on fp8 inputs ("FlashAttention v1～v4 完整进化史", v3 part 3: both
 * products on fp8 matrix cores, with block scales): q8, k8, v8 e4m3fn codes
 * [B,H,N,d] with scales sq, sk, sv [B,H,ceil(N/64)] as written by
 * fa_quant_fp8 with the same block_rows (64: one scale per 64-row block;
 * 0: one per-tensor scale, broadcast to every entry); the dequantised value
 * of a code is decode(code) * s of its 64-row block. Other block_rows give
 * FA_ERR_UNSUPPORTED: the kernel's key tile is one 64-row scale block. Keys are taken
 * in tiles of 64 (one scale block each); after each tile the row's
 * reference m is its running maximum rounded up to a whole power of two
 * (m = ln2 * an integer; the lazy rescaling of v4 part 3), P~ = exp(S - m)
 * <= 1 is rounded to e4m3 as
 * e4m3(P~ * 448) for the product with V (dequantised by sv / 448 of its
 * tile), and the row sum l uses the float32 P~. Both products run on fp8
 * matrix cores into float32 accumulators; the V block scale enters the
 * product with P as the instruction's exponent scale, so sv entries must be
 * powers of two in [2^-126, 2^127] (fa_quant_fp8 with pow2 = 1 writes
 * them): every 256-row query tile whose key range includes a tile with any
 * other sv comes out NaN (O and LSE), since the device data is not read
 * before the launch. sq and sk
 * (either form) must be positive and finite.
 * o: [B,H,N,d] bf16 (written). lse: [B,H,N] float32 (written). d must be
 * 128. */
FA_API int fa_fwd_fp8(const unsigned char* q8, const unsigned char* k8, const unsigned char* v8,
               const float* sq, const float* sk, const float* sv, int block_rows,
               void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/* Decoding of fp8 codes: out = decode(x8) * s of the code's 64-row block
 * (x8, scales as fa_quant_fp8 writes them with the same block_rows, 64 or
 * 0), rounded to bf16; out: [B,H,N,d] bf16 (written). Exact when s is a
 * power of two and the product stays in bf16's range. A block whose scale is
 * not a power of two in [2^-126, 2^127] is written as NaN (the device data
 * is not read before the launch). */
FA_API int fa_dequant_fp8(const unsigned char* x8, const float* scales, int block_rows, void* out,
                   int B, int H, int N, int d, void* stream);

/* Workspace bytes fa_bwd_fp8 needs: fa_bwd_workspace_bytes plus three
 * decoded [B,H,N,d] bf16 tensors (each 256-byte aligned); 0 for invalid
 * sizes. */
FA_API size_t fa_bwd_fp8_workspace_bytes(int B, int H, int N, int d);

/* Backward of the fp8 forward. The pages put fp8 in the forward only
 * ("FlashAttention v1～v4 完整进化史", v3 part 3); this library's reading:
 * the codes and scales are the inputs, so no gradient flows through the
 * rounding, and dq, dk, dv are the gradients with respect to the dequantised
 * Q, K, V, formed by the backward step of "6.1 FlashAttention V1详解"
 * (sections 6.1-6.2) from fa_fwd_fp8's saved o and lse: P = exp(S - L) with
 * the scores of the dequantised inputs, D = rowsum(dout * o). All three
 * tensors must be quantised with power-of-two scales (fa_quant_fp8 with
 * pow2 = 1): the call decodes them into bf16 in the workspace, exactly for
 * such scales, and runs the bf16 backward (fa_bwd) on them; a block with any
 * other scale decodes to NaN and so do the gradients it reaches.
 * q8, k8, v8: [B,H,N,d] codes; sq, sk, sv: [B,H,ceil(N/64)] scales with
 * block_rows 64 or 0; o: [B,H,N,d] bf16 and lse: [B,H,N] float32 from
 * fa_fwd_fp8; dout: [B,H,N,d] bf16; dq, dk, dv: [B,H,N,d] bf16 (written);
 * workspace: >= fa_bwd_fp8_workspace_bytes bytes, 256-byte aligned,
 * overwritten. d must be 64 or 128. */
FA_API int fa_bwd_fp8(const unsigned char* q8, const unsigned char* k8, const unsigned char* v8,
               const float* sq, const float* sk, const float* sv, int block_rows,
               const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/* Static text for a status code. */
FA_API const char* fa_status_string(int status);

/* Thread-local description of the last non-OK return on this thread ("" if none). */
FA_API const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
