/*
 * attn.h — exact scaled-dot-product attention forward on AMD Instinct MI355X
 * (gfx950), as a C ABI.
 *
 * The operation.  For every (batch, head), or every (sequence, head) of a
 * variable-length batch:
 *
 *     S   = scale * Q K^T                      [Nq, Nk]
 *     S_ij = -inf where causal and j > i       (top-left: key j is visible to
 *                                               query i iff j <= i)
 *     O   = softmax_rows(S) V                  [Nq, d]
 *     lse_i = log sum_j exp(S_ij)              (natural log)
 *
 * Standard attention materialises S ("Flash Attention 3：让 GPU 跑满的注意力
 * 计算", §1.2).  This library never does: each workgroup owns a block of
 * queries, streams K and V through LDS tile by tile, and keeps the running
 * row maximum, the running row sum and a rescaled fp32 output accumulator in
 * registers (the online-softmax recurrence of the same page, §2.2, with the
 * one-workgroup-per-query-block decomposition of §3.1).  The result is exact
 * attention up to floating-point rounding ("FlashAttention-3", opening
 * paragraph: exact attention).  lse is not on the pages; it is what a caller
 * needs to merge partial results over key shards.
 *
 * Ownership and behaviour (all entry points):
 *   - every array argument is a DEVICE pointer owned by the caller; the
 *     library allocates nothing, keeps no pointer after it returns, and holds
 *     no state between calls (thread-safe);
 *   - work is enqueued on the given HIP stream (attn_fwd: the null stream) and
 *     the host is never synchronised;
 *   - the return value is the only error channel: ATTN_OK or a negative code.
 *     Argument validation happens before any HIP call, so a bad call is
 *     rejected without touching the device.  attn_strerror() names a code.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_DT_F16 = 0,      /* IEEE binary16 */
  ATTN_DT_BF16 = 1,     /* bfloat16 */
  ATTN_DT_FP8_E4M3 = 2, /* OCP e4m3fn codes (uint8), with fp32 block scales */
  ATTN_DT_F32 = 3,      /* float32: only as the input of attn_fp8_quantize */
  ATTN_DT_INT8 = 4      /* signed 8-bit codes: only as an attn_fwd_paged cache */
} attn_dtype_t;

enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, bad flag, bad scale */
  ATTN_ERR_UNSUPPORTED = -2, /* valid request this build does not implement (e.g. d = 96) */
  ATTN_ERR_HIP = -3,         /* the HIP runtime reported an error at launch */
  ATTN_ERR_TOO_LARGE = -4    /* attn_fwd_splitkv_noalloc: the partial outputs exceed its fixed scratch */
};

/*
 * attn_fwd — O = softmax(scale Q K^T [+causal]) V and lse, on the null stream.
 *
 * Layouts (row-major, contiguous, no strides):
 *   dense   (cu_seqlens_q == cu_seqlens_k == NULL):
 *           q [B, H, Nq, d]; k, v [B, H, Nk, d]; o [B, H, Nq, d]; lse [B, H, Nq]
 *   varlen  (both cu_seqlens non-NULL; "Flash Attention 3：让 GPU 跑满的注意力
 *           计算", §5.2): B sequences packed along the token axis with no
 *           padding; cu_seqlens_q/k are int32 device arrays of B+1 cumulative
 *           lengths [0, L0, L0+L1, ...]; Nq, Nk are the total packed tokens;
 *           q [H, Nq, d]; k, v [H, Nk, d]; o [H, Nq, d]; lse [H, Nq].
 *           Sequence b uses rows [cu_q[b], cu_q[b+1]) of q and
 *           [cu_k[b], cu_k[b+1]) of k, v; causal uses indices local to the
 *           sequence.  The kernel clamps cu_seqlens into [0, N] and never
 *           faults on inconsistent values (the result is then unspecified).
 *
 * dtype: ATTN_DT_F16 / ATTN_DT_BF16: q, k, v, o all of that type; the two
 *   products run on MFMA with fp32 accumulation, all softmax arithmetic is
 *   fp32.  ATTN_DT_FP8_E4M3: q, k, v are e4m3 codes (uint8) as written by
 *   attn_fp8_quantize, o is bfloat16, and q_scale, k_scale, v_scale are the
 *   fp32 dequantisation multipliers [B, H, ceil(N/128)] (one per 128-row
 *   tile; "FlashAttention-3", "Three techniques" §3: block quantisation).
 *   fp8 varlen: the tiles restart at every sequence, so no tile spans two
 *   sequences; the scales are [H, ceil(N/128) + B] with tile j of sequence b
 *   at entry floor(cu_seqlens[b] / 128) + b + j (the layout
 *   attn_fp8_quantize_varlen writes; entries no tile owns are not read).
 *   For fp16/bf16 the three scale pointers are ignored (may be NULL); for
 *   fp8 they may be NULL only where the tensor is empty (Nq or Nk = 0).
 *   Scales must be >= 0 (attn_fp8_quantize writes positive ones).  A V
 *   tile whose scale is 0 (or so small against the head's largest V scale
 *   that its rounded weights are all 0) adds nothing to O but its keys still
 *   count in the softmax sum.
 *
 * d ∈ {64, 128, 256} (else ATTN_ERR_UNSUPPORTED), fp8 included.
 * scale: finite and >= 0 (typically 1/sqrt(d)).  causal ∈ {0, 1}.
 * B, H >= 1; Nq, Nk >= 0.  Nq = 0 is a no-op; Nk = 0 (or an empty key
 * sequence) gives O = 0 and lse = -inf.  q, o, lse may be NULL only if
 * Nq = 0, and k, v only if Nk = 0.  Pointers must be 16-byte aligned
 * (cu_seqlens and the scales: 4-byte).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Nq, int Nk, int d, float scale, int causal,
             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
             const float* q_scale, const float* k_scale, const float* v_scale);

/* attn_fwd_stream — attn_fwd on the HIP stream `hip_stream` (a hipStream_t;
 * NULL = the null stream).  Same arguments, layouts and errors as attn_fwd. */
int attn_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
                    const float* q_scale, const float* k_scale, const float* v_scale,
                    void* hip_stream);

/*
 * attn_fp8_quantize — the fp8 pre-processing of one tensor
 * ("FlashAttention-3", "Three techniques" §3 FP8 precision).
 *
 *   x [B, H, N, d] of x_dtype (ATTN_DT_F32, ATTN_DT_BF16 or ATTN_DT_F16).
 *   If signs != NULL (fp32 [d], each +1 or -1): incoherent processing first,
 *     x' = x diag(signs) H_d / sqrt(d), with H_d the Sylvester Hadamard
 *     matrix applied along d by a fast Walsh-Hadamard transform (used for Q
 *     and K; V is passed with signs == NULL).
 *   Then block quantisation: for every (b, h, 128-row tile) t,
 *     s_t = amax_t / 448 (s_t = 1 if the tile is all zero; s_t = 2^-149,
 *     the smallest positive fp32, where amax_t / 448 underflows), with amax
 *     over the tile's rotated values, and x_fp8 = e4m3(x' / s_t) rounded to
 *     nearest-even in fp32; x' ~= s_t * x_fp8.
 *   per_tensor = 1 replaces the per-tile amax by one amax over the whole
 *     tensor (every entry of x_scale then holds the same s): the per-tensor
 *     fp8 baseline the block scheme is compared with.
 *   Outputs: x_fp8 uint8 [B, H, N, d]; x_scale fp32 [B, H, ceil(N/128)].
 *   d ∈ {64, 128, 256}.  N = 0 is a no-op.  Same pointer, stream and error
 *   rules as attn_fwd_stream.
 */
int attn_fp8_quantize(const void* x, int x_dtype, void* x_fp8, float* x_scale,
                      int B, int H, int N, int d, const float* signs, int per_tensor,
                      void* hip_stream);

/*
 * attn_fp8_quantize_varlen — attn_fp8_quantize for a variable-length batch
 * ("Flash Attention 3：让 GPU 跑满的注意力计算", §5.2 packed sequences with
 * cu_seqlens; "FlashAttention-3", "Three techniques" §3 block quantisation).
 *
 *   x [H, T, d] of x_dtype: nseq sequences packed along the token axis,
 *     sequence b on tokens [cu_seqlens[b], cu_seqlens[b+1]) (int32 device
 *     array of nseq+1 cumulative lengths; clamped into [0, T]).
 *   Rotation (signs) and quantisation as attn_fp8_quantize, with the
 *     128-row tiles restarting at every sequence: a tile never spans two
 *     sequences, as the attention kernel reads one scale per (sequence,
 *     128-row tile).
 *   Outputs: x_fp8 uint8 [H, T, d]; x_scale fp32 [H, ceil(T/128) + nseq]
 *     (a size that needs no sequence lengths on the host): tile j of
 *     sequence b at entry floor(cu_seqlens[b] / 128) + b + j, so a reader
 *     finds a sequence's scales from its first token alone (these ranges
 *     never overlap and end below floor(T/128) + nseq); the entries no tile
 *     owns are written too (1, or the tensor scale with per_tensor = 1) and
 *     never read.
 *   H, nseq >= 1; T >= 0 (T = 0 is a no-op).  cu_seqlens must be non-NULL.
 *   Same pointer, stream and error rules as attn_fp8_quantize.
 */
int attn_fp8_quantize_varlen(const void* x, int x_dtype, void* x_fp8, float* x_scale,
                             int H, int T, int d, const int32_t* cu_seqlens, int nseq,
                             const float* signs, int per_tensor, void* hip_stream);

/*
 * attn_fwd_splitkv — attn_fwd (dense layout only) computed over key chunks
 * and merged: the keys of every (b, h) are cut into num_splits chunks of
 * ceil(Nk / num_splits) rows; each (b, h, chunk, query tile) is an
 * independent work item, which writes the chunk's normalised output and its
 * lse in fp32 to the workspace; attn_merge then combines them into o, lse.
 * This is FlashDecoding ("FlashAttention-3" wiki page, related work): with
 * few queries (decoding: Nq = 1 per head) the key length, not the query
 * count, supplies the parallelism.  Causal masks use absolute key indices
 * (same top-left convention as attn_fwd); a chunk that a query cannot see
 * contributes nothing.  The result equals attn_fwd's up to rounding.
 *
 *   dtype ATTN_DT_F16 or ATTN_DT_BF16 (fp8: ATTN_ERR_UNSUPPORTED; see
 *     attn_fwd_splitkv_fp8);
 *   1 <= num_splits <= 1024 (more chunks than keys is allowed: the extra
 *     chunks are empty);
 *   o_part: fp32 workspace [num_splits, B, H, Nq, d], lse_part: fp32
 *     [num_splits, B, H, Nq], both caller-owned, 16- and 4-byte aligned; on
 *     return they hold the per-chunk results (O_s normalised, lse_s = -inf
 *     for a chunk with no visible key).  NULL only if Nq = 0.
 * Other arguments, layouts and errors as attn_fwd_stream (no cu_seqlens).
 */
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                     int num_splits, float* o_part, float* lse_part, void* hip_stream);

/*
 * attn_fwd_splitkv_noalloc — attn_fwd_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without o_part and
 * lse_part, the same result (the same kernels and key chunks).  The
 * partial outputs go to a fixed device array inside the library,
 * ATTN_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs on
 * holds until the process ends; the call itself allocates nothing (its first
 * call on a device looks the array's address up once).
 *
 *   Needs num_splits * B * H * Nq * (d + 1) * 4 bytes (the O parts rounded
 *   up to 256 bytes) <= ATTN_NOALLOC_SCRATCH_BYTES, else ATTN_ERR_TOO_LARGE
 *   (nothing is launched).  Other errors as attn_fwd_splitkv.
 *   Every call on one GPU uses the same array: calls that overlap in time on
 *   one GPU (two streams, two host threads) race and give wrong results;
 *   calls on one stream are ordered and safe.  Nothing in the array needs
 *   to be cleared between calls (every entry read is written first).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                             int num_splits, void* hip_stream);

/*
 * attn_fwd_splitkv_fp8 — attn_fwd_splitkv on the fp8 operands of attn_fwd
 * (ATTN_DT_FP8_E4M3: e4m3 codes q8, k8, v8 with their per-128-row-tile fp32
 * scales [B, H, ceil(N/128)], as attn_fp8_quantize writes them; dense
 * layout): FlashDecoding ("FlashAttention-3" wiki page, related work) on the
 * block-quantised fp8 attention ("Three techniques" §3 of that page).  The
 * keys of every (b, h) are cut into num_splits chunks of ceil(Nk /
 * num_splits) keys rounded up to whole 128-row scale tiles (the last chunks
 * may be short or empty); each chunk is the fp8 attention of its keys alone
 * (its own largest V scale for the P weights, a running max that starts at
 * the chunk), causal masks with absolute key indices (top-left); the
 * chunks' normalised O and lse go to the fp32 workspace and attn_merge
 * combines them into o (bfloat16) and lse.
 *   q8 [B, H, Nq, d], k8, v8 [B, H, Nk, d] uint8 codes; q_scale [B, H,
 *   ceil(Nq/128)], k_scale, v_scale [B, H, ceil(Nk/128)] fp32 >= 0;
 *   o bfloat16 [B, H, Nq, d]; lse fp32 [B, H, Nq]; o_part fp32
 *   [num_splits, B, H, Nq, d], lse_part fp32 [num_splits, B, H, Nq]
 *   (caller-owned workspace, as attn_fwd_splitkv).  d ∈ {64, 128, 256};
 *   1 <= num_splits <= 1024.  Pointer, alignment, NULL (only for empty
 *   tensors), stream and error rules as attn_fwd_stream with fp8 operands.
 */
int attn_fwd_splitkv_fp8(const void* q8, const float* q_scale, const void* k8, const float* k_scale, const void* v8,
                         const float* v_scale, void* o, float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                         int causal, int num_splits, float* o_part, float* lse_part, void* hip_stream);

/*
 * attn_merge — combine results over disjoint key chunks (the online-softmax
 * combination of "Flash Attention 3：让 GPU 跑满的注意力计算", §2.2, for any
 * number of blocks):
 *     lse = ln sum_s e^{lse_s},    O = sum_s e^{lse_s - lse} O_s,
 * with lse_s = -inf parts ignored; a row whose parts are all -inf gives
 * O = 0 and lse = -inf.  This is also the merge of results computed on
 * different devices over key shards.
 *   o_part fp32 [num_splits, B, H, Nq, d] (normalised rows), lse_part fp32
 *   [num_splits, B, H, Nq]; o [B, H, Nq, d] of o_dtype (ATTN_DT_F16 or
 *   ATTN_DT_BF16); lse fp32 [B, H, Nq].  1 <= num_splits <= 1024,
 *   d ∈ {64, 128, 256}; 16-byte aligned arrays (lse arrays: 4-byte).
 *   Nq = 0 is a no-op.  Same stream and error rules as attn_fwd_stream.
 */
int attn_merge(const float* o_part, const float* lse_part, int num_splits, int B, int H, int Nq, int d,
               void* o, float* lse, int o_dtype, void* hip_stream);

/*
 * attn_fwd_paged — attention of dense queries over a paged key/value cache
 * ("Flash Attention 3：让 GPU 跑满的注意力计算", §5.3: the method run on the
 * pages of a PagedAttention cache; here the kernel reads each tile from its
 * page through the table, no contiguous copy is made), computed over
 * `num_splits` key chunks and merged as attn_fwd_splitkv.  Non-causal: every
 * query of sequence b attends to all its seqlens_k[b] cached keys (the
 * decoding setting).  The cache may hold 8-bit codes (INT8 and FP8 KV
 * caches, §4.1.3 of the same post).
 *   q [B, H, Nq, d]; o [B, H, Nq, d] (same dtype, ATTN_DT_F16/BF16);
 *   lse fp32 [B, H, Nq];
 *   k_cache, v_cache [num_pages, page_size, H, d]: row (page, i, h) holds
 *     head h of one token; of type kv_dtype: `dtype` (16-bit cache, k_scale
 *     and v_scale ignored), ATTN_DT_FP8_E4M3 (OCP e4m3fn codes) or
 *     ATTN_DT_INT8 (signed codes);
 *   k_scale, v_scale fp32 [num_pages, page_size, H] (8-bit caches): the
 *     cached key/value of a (token, head) is scale * decode(code);
 *   block_table int32 [B, max_pages]: token t of sequence b is row
 *     t % page_size of page block_table[b][t / page_size];
 *   seqlens_k int32 [B]: keys of each sequence (clamped to
 *     [0, max_pages * page_size]; 0 gives O = 0, lse = -inf);
 *   page indices outside [0, num_pages) are clamped (never read out of
 *     bounds; the result is then unspecified);
 *   page_size a multiple of 64 (else ATTN_ERR_UNSUPPORTED);
 *   o_part fp32 [num_splits, B, H, Nq, d], lse_part fp32 [num_splits, B, H,
 *     Nq]: caller-owned workspace, as attn_fwd_splitkv (chunks of
 *     ceil(max_pages * page_size / num_splits) keys rounded up to 64).
 *   All device pointers; tensors 16-byte aligned, int32 and lse arrays
 *   4-byte aligned; NULL allowed only when Nq = 0.  fp8 queries:
 *   UNSUPPORTED here (attn_fwd_paged_fp8 takes them).  Same stream and
 *   error rules as attn_fwd_stream.
 */
int attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                   const float* v_scale, const int32_t* block_table, const int32_t* seqlens_k, void* o, float* lse,
                   int B, int H, int Nq, int d, int num_pages, int page_size, int max_pages, float scale, int dtype,
                   int kv_dtype, int num_splits, float* o_part, float* lse_part, void* hip_stream);

/*
 * attn_fwd_paged_fp8 — attn_fwd_paged with e4m3 queries over an 8-bit
 * cache, for decoding: one or two query rows per (batch, head) (FP8
 * attention, "FlashAttention-3" wiki page, "Three techniques" §3, with the
 * INT8 / FP8 KV caches of "Flash Attention 3：让 GPU 跑满的注意力计算",
 * §4.1.3).
 *   q [B, H, Nq, d]: OCP e4m3fn codes; q_scale fp32 [B, H]: query row i of
 *     (b, h) is q_scale[b][h] * decode(code) (the per-128-row tile scale of
 *     attn_fwd's fp8 layout [B, H, ceil(Nq / 128)] for Nq <= 128);
 *   Nq in [0, 2]; more query rows: ATTN_ERR_UNSUPPORTED;
 *   kv_dtype ATTN_DT_FP8_E4M3 or ATTN_DT_INT8 (else ATTN_ERR_INVALID_ARG),
 *     with k_scale and v_scale as attn_fwd_paged;
 *   o bf16 [B, H, Nq, d]; every other argument, the workspace, ownership and
 *     the error rules as attn_fwd_paged.
 */
int attn_fwd_paged_fp8(const void* q, const float* q_scale, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* block_table,
                       const int32_t* seqlens_k, void* o, float* lse, int B, int H, int Nq, int d, int num_pages,
                       int page_size, int max_pages, float scale, int kv_dtype, int num_splits, float* o_part,
                       float* lse_part, void* hip_stream);

/*
 * attn_bwd — gradients of the attention computed by attn_fwd: given dO =
 * dL/dO, writes dQ, dK, dV (the derivative of the forward definition of
 * "Flash Attention 3：让 GPU 跑满的注意力计算", §1.2 and §2.2; the
 * "FlashAttention-3" wiki page measures such a backward pass in its
 * "Measured (H100 80GB SXM5)" table):
 *     dV = P^T dO,  dS = P * (dO V^T - delta),  delta_i = dO_i . O_i,
 *     dQ = scale dS K,  dK = scale dS^T Q.
 * P is recomputed from Q, K and the forward's lse; no N x N matrix is
 * stored.
 *   q, o, dout, dq [B, H, Nq, d]; k, v, dk, dv [B, H, Nk, d]; all of dtype
 *     ATTN_DT_F16 or ATTN_DT_BF16, contiguous, 16-byte aligned;
 *   cu_seqlens_q / cu_seqlens_k: NULL (dense) or, both, int32 [B+1] prefix
 *     sums as in attn_fwd: then q, o, dout, dq are [H, Nq, d], k, v, dk, dv
 *     [H, Nk, d], lse and delta [H, Nq] over B packed sequences (causal
 *     masks per sequence, local indices);
 *   o, lse: the forward's outputs for the same q, k, v, scale, causal;
 *   delta: fp32 workspace [B, H, Nq], caller-owned, 4-byte aligned; on
 *     return it holds delta_i = sum_c dO_ic O_ic;
 *   d ∈ {64, 128, 256} (fp8: ATTN_ERR_UNSUPPORTED).
 *   Query-side arrays may be NULL only if Nq = 0, key-side arrays only if
 *   Nk = 0.  Nk = 0 gives dQ = 0; Nq = 0 gives dK = dV = 0.  dQ is
 *   accumulated per query row in one workgroup (no atomics): results are
 *   deterministic.  Same stream, ownership and error rules as
 *   attn_fwd_stream.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, float* delta, int B, int H, int Nq, int Nk, int d, float scale,
             int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype, void* hip_stream);

/*
 * attn_bwd_fp8 — attn_bwd on the fp8 operands of attn_fwd (dtype
 * ATTN_DT_FP8_E4M3, d = 128, dense layout), with E5M2 for the gradient
 * operands ("Flash Attention 3：让 GPU 跑满的注意力计算", §4.1.2: E4M3 for the
 * forward pass, E5M2 for back-propagation).  The gradients are those of the
 * attention of the dequantised inputs q = q_scale[tile] * e4m3(q8) etc.
 * (for inputs that attn_fp8_quantize rotated: with respect to the rotated
 * Q and K), the five products on fp8 matrix cores with fp32 accumulation:
 *   dO is quantised to e5m2 with one fp32 scale per 128-row tile,
 *     s = amax / 57344 (1 for an all-zero tile), codes e5m2(dO / s);
 *   dV = P^T dO takes P as e4m3(2^8 P s_do(q) / max s_do);
 *   dK = scale dS^T Q takes dS as e5m2(dS s_q(q) / max s_q);
 *   dQ = scale dS K takes dS as e5m2(dS s_k(k) / max s_k);
 *   (max over the (b, h)'s tiles: each product's per-tile scale is folded
 *   into the factor that is rounded); P = exp(S - lse) from the
 *   dequantised scores, dP = dO_q V^T, dS = P (dP - delta), delta_i =
 *   dO_i . O_i in fp32 from the unquantised dO.  Rounding: to nearest even;
 *   e5m2 values saturate at +-57344.
 *   q8 uint8 [B, H, Nq, 128], k8, v8 uint8 [B, H, Nk, 128] and q_scale,
 *     k_scale, v_scale fp32 [B, H, ceil(N/128)]: attn_fwd's fp8 inputs;
 *   o (bfloat16 [B, H, Nq, 128]) and lse (fp32 [B, H, Nq]): attn_fwd's
 *     outputs for the same inputs, scale and causal;
 *   dout bfloat16 [B, H, Nq, 128]; dq, dk, dv bfloat16, shaped as q8, k8, v8;
 *   workspaces, caller-owned, overwritten: stats fp32 [3, B, H, Nq] (on
 *     return lse_i log2(e), delta_i, and delta_i s_q(tile) / max s_q), do8
 *     uint8 [B, H, Nq, 128] (dO's e5m2 codes) and do_scale fp32
 *     [B, H, ceil(Nq/128)] (their scales);
 *   d other than 128: ATTN_ERR_UNSUPPORTED.  2-D arrays 16-byte aligned,
 *   lse, scales, delta 4-byte aligned.
 *   Query-side arrays may be NULL only if Nq = 0, key-side arrays only if
 *   Nk = 0.  Nk = 0 gives dQ = 0; Nq = 0 gives dK = dV = 0.  No atomics:
 *   results are deterministic.  Same stream, ownership and error rules as
 *   attn_fwd_stream.
 */
int attn_bwd_fp8(const void* q8, const float* q_scale, const void* k8, const float* k_scale, const void* v8,
                 const float* v_scale, const void* o, const float* lse, const void* dout, void* dq, void* dk,
                 void* dv, float* stats, void* do8, float* do_scale, int B, int H, int Nq, int Nk, int d,
                 float scale, int causal, void* hip_stream);

/* attn_strerror — a static, human-readable name for a return code. */
const char* attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
