// Host/device parameter blocks of the attention kernels and the internal
// launch entry points the C ABI dispatches to.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Nq, Nk;
  float c;               // scale * log2(e): scores are handled in base 2
  const int32_t* cu_q;   // varlen only
  const int32_t* cu_k;   // varlen only
  int tiles_per_head;    // query tiles per (b, h) (varlen: upper bound per head)
  int n_work;            // work items (workgroups launched, unless persistent)
  int queue;             // persistent launches: the work-queue slot of this launch
  int pair_tiles;        // dense: each workgroup runs query tiles t and T-1-t (set by the launch)
  const float* q_scale;  // fp8 only: [B, H, ceil(Nq/128)]; varlen [H, ceil(Nq/128) + B]
  const float* k_scale;  // fp8: [B, H, ceil(Nk/128)] (varlen [H, ceil(Nk/128) + B]); 8-bit paged cache: [num_pages, page_size, H]
  const float* v_scale;
  int n_split;           // key chunks (split launches only)
  int split_len;         // keys per chunk
  float* o_part;         // [n_split, B, H, Nq, d] fp32 normalised partial outputs
  float* lse_part;       // [n_split, B, H, Nq]
  // paged key/value cache (split launches only): K and V rows of token t of
  // sequence b, head h at cache[block_table[b * max_pages + t / page_size],
  // t % page_size, h] of a [num_pages, page_size, H, d] array
  const int32_t* block_table;  // [B, max_pages]
  const int32_t* seqlens_k;    // [B]
  int page_size;
  int max_pages;
  int num_pages;
};

struct MergeParams {
  const float* o_part;   // [S, rows, d]
  const float* lse_part; // [S, rows]
  int S;
  int64_t rows;          // B * H * Nq
  int d;
  void* o;               // [rows, d] in o_dtype (fp16 or bf16)
  int o_dtype;
  float* lse;            // [rows]
};

struct PrepParams {
  const void* x;
  int x_dtype;           // attn_dtype_t of x
  uint8_t* x8;
  float* scale;          // [B, H, ceil(N/128)]
  int BH, N, d;
  const float* signs;    // NULL: no rotation
  int mode;              // 0: block scales; 1: tile amax only; 2: quantise with the tensor amax
  // variable-length batch (cu non-NULL): x is [H, N, d] with sequence s on
  // tokens [cu[s], cu[s+1]); scale is [H, ceil(N/128) + nseq], tile j of
  // sequence s at entry floor(cu[s] / 128) + s + j
  const int32_t* cu;
  int nseq;
};

// Query rows per workgroup of each kernel variant (sizes the grid).
// Backward pass (fp16/bf16, dense [B, H, N, d]).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;          // [B, H, Nq] fp32: rowsum(dO * O), written by the first kernel
  int B, H, Nq, Nk;
  float scale;           // softmax scale (multiplies dS in dQ and dK)
  float c;               // scale * log2(e)
  int tiles_per_head;    // set per launch: key tiles (dK/dV) or query tiles (dQ) per head
  int n_work;
  const int32_t* cu_q;   // varlen only: [B+1] prefix sums over the packed tokens
  const int32_t* cu_k;
};

// Backward pass on fp8 operands (dense [B, H, N, 128]).
struct Bwd8Params {
  const uint8_t* q;      // e4m3 codes and their per-128-row-tile scales [B, H, ceil(N/128)]
  const uint8_t* k;
  const uint8_t* v;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const void* o;         // bfloat16 [B, H, Nq, 128]: the forward's output
  const void* dout;      // bfloat16 [B, H, Nq, 128]
  const float* lse;      // [B, H, Nq]
  float* stats;          // workspace [3, B, H, Nq]: lse log2(e); delta = rowsum(dO * O); delta s_q(tile) / max s_q
  uint8_t* do8;          // workspace [B, H, Nq, 128]: e5m2 codes of dO
  float* do_scale;       // workspace [B, H, ceil(Nq/128)]
  void* dq;              // bfloat16 outputs
  void* dk;
  void* dv;
  int B, H, Nq, Nk;
  float scale;           // softmax scale
  float c;               // scale * log2(e)
  int n_work;            // workgroups of the current launch
};
hipError_t launch_bwd_fp8(bool causal, const Bwd8Params& p, hipStream_t st);

int bwd_key_block(int d);    // keys per dK/dV workgroup
int bwd_query_block(int d);  // queries per dQ workgroup
hipError_t launch_bwd(int dtype, int d, bool causal, bool varlen, BwdParams p, hipStream_t st);

// Argument checks of attn_fwd_splitkv (host only): ATTN_OK or an error code.
int validate_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                     int d, float scale, int causal, int dtype, int num_splits, const float* o_part,
                     const float* lse_part);

int fwd_block_rows(int dtype, int d, bool causal, bool varlen);
int fwd_split_block_rows(int dtype, int d, bool causal);  // key-chunk launches
int fwd_split_tile_keys(int d);  // key rows per tile of key-chunk launches (chunk lengths are multiples)
int fwd_fp8_block_rows(bool causal);

// kv: 0 dense K/V, 1 paged 16-bit cache, 2 paged e4m3 cache, 3 paged int8
// cache (8-bit caches: per-(token, head) scales in k_scale / v_scale)
hipError_t launch_fwd(int dtype, int d, bool causal, bool varlen, bool split, int kv, const FwdParams& p,
                      hipStream_t st);
hipError_t launch_merge(const MergeParams& p, hipStream_t st);
// Key-chunk launches with at most kDecodeMaxRows query rows per head over
// dense K/V or an 8-bit paged cache (decode_shape) run the decoding-shaped
// kernel (attn_decode.hip); kv as launch_fwd, causal only with dense K/V.
// Measured against the prefill kernel's key-chunk launches (B2 H32 Nk32768
// d128): 1 row 190 vs 195 us dense, 137 vs 186 us on an e4m3 paged cache;
// slower from 4 rows and on a 16-bit paged cache (210 vs 204 us).
constexpr int kDecodeMaxRows = 2;
bool decode_shape(int Nq, int kv);
hipError_t launch_decode(int dtype, int d, bool causal, int kv, const FwdParams& p, hipStream_t st);
// split: key chunks of p.split_len keys (a multiple of 128), per-chunk results
// to p.o_part / p.lse_part as the 16-bit key-chunk launch
hipError_t launch_fwd_fp8(int d, bool causal, bool varlen, bool split, const FwdParams& p, hipStream_t st);
hipError_t launch_fp8_prep(const PrepParams& p, bool per_tensor, hipStream_t st);

}  // namespace attn
