// The C ABI of include/attn.h: argument validation (pure host code, before
// any HIP call), variant dispatch and launch geometry.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/attn.h"
#include "attn_params.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool supported_d(int d) { return d == 64 || d == 128 || d == 256; }

constexpr int kMaxSplits = 1024;  // key chunks per split-KV call

// Validation shared by attn_fwd and attn_fwd_stream.  Returns ATTN_OK or an
// error code; touches no device state.
int validate_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                 int d, float scale, int causal, const int32_t* cu_q, const int32_t* cu_k, int dtype,
                 const float* q_scale, const float* k_scale, const float* v_scale) {
  if (B < 1 || H < 1 || Nq < 0 || Nk < 0) return ATTN_ERR_INVALID_ARG;
  // q, o, lse may be NULL only when there are no queries; k, v only when there are no keys
  if (Nq > 0 && (!q || !o || !lse)) return ATTN_ERR_INVALID_ARG;
  if (Nk > 0 && (!k || !v)) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if ((cu_q == nullptr) != (cu_k == nullptr)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DT_F16 && dtype != ATTN_DT_BF16 && dtype != ATTN_DT_FP8_E4M3) return ATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return ATTN_ERR_INVALID_ARG;
  if (cu_q && (!aligned(cu_q, 4) || !aligned(cu_k, 4))) return ATTN_ERR_INVALID_ARG;
  if (dtype == ATTN_DT_FP8_E4M3) {
    // scales may be NULL only for an empty tensor, like the tensor itself
    if ((Nq > 0 && !q_scale) || (Nk > 0 && (!k_scale || !v_scale))) return ATTN_ERR_INVALID_ARG;
    if (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4)) return ATTN_ERR_INVALID_ARG;
  }
  if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
  if (cu_q == nullptr && (int64_t)B * H > (int64_t)INT32_MAX / 2) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

}  // namespace

namespace attn {

int validate_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                     int d, float scale, int causal, int dtype, int num_splits, const float* o_part,
                     const float* lse_part) {
  // fp8 is not offered here: validate the rest as for bf16, then refuse it
  const int vdt = dtype == ATTN_DT_FP8_E4M3 ? ATTN_DT_BF16 : dtype;
  const int rc = validate_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, nullptr, nullptr, vdt, nullptr,
                              nullptr, nullptr);
  if (rc != ATTN_OK) return rc;
  if (num_splits < 1 || num_splits > kMaxSplits) return ATTN_ERR_INVALID_ARG;
  if (Nq > 0 && (!o_part || !lse_part)) return ATTN_ERR_INVALID_ARG;
  if (!aligned(o_part, 16) || !aligned(lse_part, 4)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DT_F16 && dtype != ATTN_DT_BF16) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

}  // namespace attn

extern "C" {

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: unsupported configuration";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: HIP runtime error";
    case ATTN_ERR_TOO_LARGE:
      return "ATTN_ERR_TOO_LARGE: the call's partial outputs exceed the fixed device scratch "
             "(ATTN_NOALLOC_SCRATCH_BYTES) of attn_fwd_splitkv_noalloc";
    default: return "unknown attn error code";
  }
}

int attn_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                    int d, float scale, int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int dtype, const float* q_scale, const float* k_scale, const float* v_scale, void* hip_stream) {
  const int rc = validate_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, cu_seqlens_q, cu_seqlens_k, dtype,
                              q_scale, k_scale, v_scale);
  if (rc != ATTN_OK) return rc;
  if (Nq == 0) return ATTN_OK;
  const bool varlen = cu_seqlens_q != nullptr;
  const int br = attn::fwd_block_rows(dtype, d, causal != 0, varlen);

  attn::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Nq = Nq; p.Nk = Nk;
  p.c = scale * 1.4426950408889634f;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.q_scale = q_scale; p.k_scale = k_scale; p.v_scale = v_scale;
  int64_t heads, tiles;
  if (varlen) {
    // Query-tile slots per head: tile j of sequence b is slot
    // floor(cu_q[b] / BR) + b + j < floor(Nq / BR) + B; workgroups of slots
    // no tile owns exit at once.
    heads = H;
    tiles = ((int64_t)Nq + br - 1) / br + B;
  } else {
    heads = (int64_t)B * H;
    tiles = ((int64_t)Nq + br - 1) / br;
  }
  const int64_t n_work = heads * tiles;
  if (n_work > INT32_MAX || tiles > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  p.tiles_per_head = (int)tiles;
  p.n_work = (int)n_work;

  hipStream_t st = (hipStream_t)hip_stream;
  hipError_t e;
  if (dtype == ATTN_DT_FP8_E4M3)
    e = attn::launch_fwd_fp8(d, causal != 0, varlen, false, p, st);
  else
    e = attn::launch_fwd(dtype, d, causal != 0, varlen, false, 0, p, st);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int d,
             float scale, int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
             const float* q_scale, const float* k_scale, const float* v_scale) {
  return attn_fwd_stream(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, cu_seqlens_q, cu_seqlens_k, dtype,
                         q_scale, k_scale, v_scale, nullptr);
}

int attn_merge(const float* o_part, const float* lse_part, int num_splits, int B, int H, int Nq, int d, void* o,
               float* lse, int o_dtype, void* hip_stream) {
  if (B < 1 || H < 1 || Nq < 0) return ATTN_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > kMaxSplits) return ATTN_ERR_INVALID_ARG;
  if (o_dtype != ATTN_DT_F16 && o_dtype != ATTN_DT_BF16) return ATTN_ERR_INVALID_ARG;
  if (Nq > 0 && (!o_part || !lse_part || !o || !lse)) return ATTN_ERR_INVALID_ARG;
  if (!aligned(o_part, 16) || !aligned(lse_part, 4) || !aligned(o, 16) || !aligned(lse, 4))
    return ATTN_ERR_INVALID_ARG;
  if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * H > (int64_t)INT32_MAX / 2) return ATTN_ERR_INVALID_ARG;
  if (Nq == 0) return ATTN_OK;
  attn::MergeParams mp{};
  mp.o_part = o_part; mp.lse_part = lse_part; mp.S = num_splits;
  mp.rows = (int64_t)B * H * Nq; mp.d = d; mp.o = o; mp.o_dtype = o_dtype; mp.lse = lse;
  const hipError_t e = attn::launch_merge(mp, (hipStream_t)hip_stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                     int d, float scale, int causal, int dtype, int num_splits, float* o_part, float* lse_part,
                     void* hip_stream) {
  const int rc = attn::validate_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, num_splits, o_part,
                                        lse_part);
  if (rc != ATTN_OK) return rc;
  if (Nq == 0) return ATTN_OK;
  const int br = attn::fwd_split_block_rows(dtype, d, causal != 0);
  const int64_t tiles = ((int64_t)Nq + br - 1) / br;
  const int64_t n_work = (int64_t)B * H * num_splits * tiles;
  if (n_work > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  attn::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Nq = Nq; p.Nk = Nk;
  p.c = scale * 1.4426950408889634f;
  p.tiles_per_head = (int)tiles;
  p.n_work = (int)n_work;
  p.n_split = num_splits;
  p.split_len = (int)(((int64_t)Nk + num_splits - 1) / num_splits);
  p.o_part = o_part;
  p.lse_part = lse_part;
  hipStream_t st = (hipStream_t)hip_stream;
  hipError_t e = attn::launch_fwd(dtype, d, causal != 0, false, true, 0, p, st);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  return attn_merge(o_part, lse_part, num_splits, B, H, Nq, d, o, lse, dtype, hip_stream);
}

int attn_fwd_splitkv_fp8(const void* q8, const float* q_scale, const void* k8, const float* k_scale, const void* v8,
                         const float* v_scale, void* o, float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                         int causal, int num_splits, float* o_part, float* lse_part, void* hip_stream) {
  const int rc = validate_fwd(q8, k8, v8, o, lse, B, H, Nq, Nk, d, scale, causal, nullptr, nullptr,
                              ATTN_DT_FP8_E4M3, q_scale, k_scale, v_scale);
  if (rc != ATTN_OK) return rc;
  if (num_splits < 1 || num_splits > kMaxSplits) return ATTN_ERR_INVALID_ARG;
  if (Nq > 0 && (!o_part || !lse_part)) return ATTN_ERR_INVALID_ARG;
  if (!aligned(o_part, 16) || !aligned(lse_part, 4)) return ATTN_ERR_INVALID_ARG;
  if (Nq == 0) return ATTN_OK;
  const int br = attn::fwd_fp8_block_rows(causal != 0);
  const int64_t tiles = ((int64_t)Nq + br - 1) / br;
  const int64_t n_work = (int64_t)B * H * num_splits * tiles;
  if (n_work > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  // chunks of whole 128-row scale tiles
  int64_t split_len = ((int64_t)Nk + num_splits - 1) / num_splits;
  split_len = (split_len + 127) / 128 * 128;
  attn::FwdParams p{};
  p.q = q8; p.k = k8; p.v = v8; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Nq = Nq; p.Nk = Nk;
  p.c = scale * 1.4426950408889634f;
  p.q_scale = q_scale; p.k_scale = k_scale; p.v_scale = v_scale;
  p.tiles_per_head = (int)tiles;
  p.n_work = (int)n_work;
  p.n_split = num_splits;
  p.split_len = (int)split_len;
  p.o_part = o_part;
  p.lse_part = lse_part;
  hipStream_t st = (hipStream_t)hip_stream;
  const hipError_t e = attn::launch_fwd_fp8(d, causal != 0, false, true, p, st);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  return attn_merge(o_part, lse_part, num_splits, B, H, Nq, d, o, lse, ATTN_DT_BF16, hip_stream);
}

namespace {

// attn_fwd_paged (fp8q_entry false: e4m3 queries are UNSUPPORTED there, after
// the argument checks) and attn_fwd_paged_fp8 (fp8q_entry true).
int fwd_paged(bool fp8q_entry, const void* q, const float* q_scale, const void* k_cache, const void* v_cache, const float* k_scale,
              const float* v_scale, const int32_t* block_table, const int32_t* seqlens_k, void* o, float* lse, int B,
              int H, int Nq, int d, int num_pages, int page_size, int max_pages, float scale, int dtype, int kv_dtype,
              int num_splits, float* o_part, float* lse_part, void* hip_stream) {
  const bool fp8q = dtype == ATTN_DT_FP8_E4M3;
  if (B < 1 || H < 1 || Nq < 0) return ATTN_ERR_INVALID_ARG;
  if (num_pages < 1 || max_pages < 1 || page_size < 1) return ATTN_ERR_INVALID_ARG;
  if (Nq > 0 && (!q || !k_cache || !v_cache || !block_table || !seqlens_k || !o || !lse || !o_part || !lse_part))
    return ATTN_ERR_INVALID_ARG;
  if (fp8q_entry && Nq > 0 && !q_scale) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DT_F16 && dtype != ATTN_DT_BF16 && dtype != ATTN_DT_FP8_E4M3) return ATTN_ERR_INVALID_ARG;
  const bool quant = kv_dtype == ATTN_DT_FP8_E4M3 || kv_dtype == ATTN_DT_INT8;
  if (fp8q ? !quant : (kv_dtype != dtype && !quant)) return ATTN_ERR_INVALID_ARG;
  if (quant && Nq > 0 && (!k_scale || !v_scale)) return ATTN_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > kMaxSplits) return ATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(block_table, 4) || !aligned(seqlens_k, 4) || !aligned(o_part, 16) || !aligned(lse_part, 4) ||
      !aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(q_scale, 4))
    return ATTN_ERR_INVALID_ARG;
  if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
  if (fp8q != fp8q_entry) return fp8q ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID_ARG;
  // e4m3 queries run on the decoding-shaped kernel only
  if (fp8q && Nq > attn::kDecodeMaxRows) return ATTN_ERR_UNSUPPORTED;
  const int tile = attn::fwd_split_tile_keys(d);
  if (page_size % tile != 0) return ATTN_ERR_UNSUPPORTED;
  const int64_t max_keys = (int64_t)max_pages * page_size;
  if (max_keys > INT32_MAX / 2 || (int64_t)B * max_pages > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H > (int64_t)INT32_MAX / 2) return ATTN_ERR_INVALID_ARG;
  if (Nq == 0) return ATTN_OK;
  const int br = attn::fwd_split_block_rows(dtype, d, false);
  const int64_t tiles = ((int64_t)Nq + br - 1) / br;
  const int64_t n_work = (int64_t)B * H * num_splits * tiles;
  if (n_work > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  // chunks of whole tiles, so that no tile crosses a page
  int64_t split_len = (max_keys + num_splits - 1) / num_splits;
  split_len = (split_len + tile - 1) / tile * tile;
  attn::FwdParams p{};
  p.q = q; p.k = k_cache; p.v = v_cache; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Nq = Nq; p.Nk = (int)max_keys;
  p.c = scale * 1.4426950408889634f;
  p.tiles_per_head = (int)tiles;
  p.n_work = (int)n_work;
  p.n_split = num_splits;
  p.split_len = (int)split_len;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.block_table = block_table;
  p.seqlens_k = seqlens_k;
  p.page_size = page_size;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  const int kv = kv_dtype == ATTN_DT_FP8_E4M3 ? 2 : kv_dtype == ATTN_DT_INT8 ? 3 : 1;
  hipStream_t st = (hipStream_t)hip_stream;
  const hipError_t e = fp8q ? attn::launch_decode(2, d, false, kv, p, st)
                            : attn::launch_fwd(dtype, d, false, false, true, kv, p, st);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  return attn_merge(o_part, lse_part, num_splits, B, H, Nq, d, o, lse, fp8q ? ATTN_DT_BF16 : dtype, hip_stream);
}

}  // namespace

int attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                   const float* v_scale, const int32_t* block_table, const int32_t* seqlens_k, void* o, float* lse,
                   int B, int H, int Nq, int d, int num_pages, int page_size, int max_pages, float scale, int dtype,
                   int kv_dtype, int num_splits, float* o_part, float* lse_part, void* hip_stream) {
  return fwd_paged(false, q, nullptr, k_cache, v_cache, k_scale, v_scale, block_table, seqlens_k, o, lse, B, H, Nq,
                   d, num_pages, page_size, max_pages, scale, dtype, kv_dtype, num_splits, o_part, lse_part,
                   hip_stream);
}

int attn_fwd_paged_fp8(const void* q, const float* q_scale, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* block_table,
                       const int32_t* seqlens_k, void* o, float* lse, int B, int H, int Nq, int d, int num_pages,
                       int page_size, int max_pages, float scale, int kv_dtype, int num_splits, float* o_part,
                       float* lse_part, void* hip_stream) {
  return fwd_paged(true, q, q_scale, k_cache, v_cache, k_scale, v_scale, block_table, seqlens_k, o, lse, B, H, Nq,
                   d, num_pages, page_size, max_pages, scale, ATTN_DT_FP8_E4M3, kv_dtype, num_splits, o_part,
                   lse_part, hip_stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, float* delta, int B, int H, int Nq, int Nk, int d, float scale,
             int causal, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype, void* hip_stream) {
  if (B < 1 || H < 1 || Nq < 0 || Nk < 0) return ATTN_ERR_INVALID_ARG;
  // query-side arrays may be NULL only without queries, key-side ones only without keys
  if (Nq > 0 && (!q || !o || !lse || !dout || !dq || !delta)) return ATTN_ERR_INVALID_ARG;
  if (Nk > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if ((cu_seqlens_q == nullptr) != (cu_seqlens_k == nullptr)) return ATTN_ERR_INVALID_ARG;
  if (cu_seqlens_q && (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DT_F16 && dtype != ATTN_DT_BF16 && dtype != ATTN_DT_FP8_E4M3) return ATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(delta, 4))
    return ATTN_ERR_INVALID_ARG;
  if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_DT_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * H > (int64_t)INT32_MAX / 2) return ATTN_ERR_INVALID_ARG;
  const bool varlen = cu_seqlens_q != nullptr;
  const int64_t heads = varlen ? H : (int64_t)B * H;  // varlen: [H, T, d], B sequences
  const int64_t kt = ((int64_t)Nk + attn::bwd_key_block(d) - 1) / attn::bwd_key_block(d) + (varlen ? B : 0);
  const int64_t qt = ((int64_t)Nq + attn::bwd_query_block(d) - 1) / attn::bwd_query_block(d) + (varlen ? B : 0);
  if (heads * kt > INT32_MAX || heads * qt > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  if (Nq == 0 && Nk == 0) return ATTN_OK;
  attn::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv; p.delta = delta;
  p.B = B; p.H = H; p.Nq = Nq; p.Nk = Nk;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  const hipError_t e = attn::launch_bwd(dtype, d, causal != 0, varlen, p, (hipStream_t)hip_stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_bwd_fp8(const void* q8, const float* q_scale, const void* k8, const float* k_scale, const void* v8,
                 const float* v_scale, const void* o, const float* lse, const void* dout, void* dq, void* dk,
                 void* dv, float* stats, void* do8, float* do_scale, int B, int H, int Nq, int Nk, int d,
                 float scale, int causal, void* hip_stream) {
  if (B < 1 || H < 1 || Nq < 0 || Nk < 0) return ATTN_ERR_INVALID_ARG;
  if (Nq > 0 && (!q8 || !q_scale || !o || !lse || !dout || !dq || !stats || !do8 || !do_scale))
    return ATTN_ERR_INVALID_ARG;
  if (Nk > 0 && (!k8 || !k_scale || !v8 || !v_scale || !dk || !dv)) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(do8, 16))
    return ATTN_ERR_INVALID_ARG;
  if (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(lse, 4) ||
      !aligned(stats, 4) || !aligned(do_scale, 4))
    return ATTN_ERR_INVALID_ARG;
  if (d != 128) return ATTN_ERR_UNSUPPORTED;
  // workgroups: (b, h) x 128-row tiles of either side
  const int64_t heads = (int64_t)B * H;
  if (heads * (((int64_t)Nq + 127) / 128) > INT32_MAX || heads * (((int64_t)Nk + 127) / 128) > INT32_MAX)
    return ATTN_ERR_INVALID_ARG;
  if (Nq == 0 && Nk == 0) return ATTN_OK;
  attn::Bwd8Params p{};
  p.q = (const uint8_t*)q8; p.k = (const uint8_t*)k8; p.v = (const uint8_t*)v8;
  p.q_scale = q_scale; p.k_scale = k_scale; p.v_scale = v_scale;
  p.o = o; p.dout = dout; p.lse = lse;
  p.stats = stats; p.do8 = (uint8_t*)do8; p.do_scale = do_scale;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.B = B; p.H = H; p.Nq = Nq; p.Nk = Nk;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  const hipError_t e = attn::launch_bwd_fp8(causal != 0, p, (hipStream_t)hip_stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fp8_quantize(const void* x, int x_dtype, void* x_fp8, float* x_scale, int B, int H, int N, int d,
                      const float* signs, int per_tensor, void* hip_stream) {
  if (!x || !x_fp8 || !x_scale) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 0) return ATTN_ERR_INVALID_ARG;
  if (x_dtype != ATTN_DT_F32 && x_dtype != ATTN_DT_BF16 && x_dtype != ATTN_DT_F16) return ATTN_ERR_INVALID_ARG;
  if (per_tensor != 0 && per_tensor != 1) return ATTN_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(x_fp8, 16) || !aligned(x_scale, 4)) return ATTN_ERR_INVALID_ARG;
  if (signs && !aligned(signs, 4)) return ATTN_ERR_INVALID_ARG;
  if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * H > INT32_MAX / 2) return ATTN_ERR_INVALID_ARG;
  if (N == 0) return ATTN_OK;
  attn::PrepParams p{};
  p.x = x; p.x_dtype = x_dtype; p.x8 = (uint8_t*)x_fp8; p.scale = x_scale;
  p.BH = B * H; p.N = N; p.d = d; p.signs = signs; p.mode = 0;
  hipError_t e = attn::launch_fp8_prep(p, per_tensor != 0, (hipStream_t)hip_stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fp8_quantize_varlen(const void* x, int x_dtype, void* x_fp8, float* x_scale, int H, int T, int d,
                             const int32_t* cu_seqlens, int nseq, const float* signs, int per_tensor,
                             void* hip_stream) {
  if (!x || !x_fp8 || !x_scale || !cu_seqlens) return ATTN_ERR_INVALID_ARG;
  if (H < 1 || T < 0 || nseq < 1) return ATTN_ERR_INVALID_ARG;
  if (x_dtype != ATTN_DT_F32 && x_dtype != ATTN_DT_BF16 && x_dtype != ATTN_DT_F16) return ATTN_ERR_INVALID_ARG;
  if (per_tensor != 0 && per_tensor != 1) return ATTN_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(x_fp8, 16) || !aligned(x_scale, 4) || !aligned(cu_seqlens, 4))
    return ATTN_ERR_INVALID_ARG;
  if (signs && !aligned(signs, 4)) return ATTN_ERR_INVALID_ARG;
  if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
  // scale entries per head: ceil(T / 128) + nseq; the grid is H times that
  if (((int64_t)T + 127) / 128 + nseq > INT32_MAX / 2 ||
      (int64_t)H * (((int64_t)T + 127) / 128 + nseq) > INT32_MAX)
    return ATTN_ERR_INVALID_ARG;
  if (T == 0) return ATTN_OK;
  attn::PrepParams p{};
  p.x = x; p.x_dtype = x_dtype; p.x8 = (uint8_t*)x_fp8; p.scale = x_scale;
  p.BH = H; p.N = T; p.d = d; p.signs = signs; p.mode = 0;
  p.cu = cu_seqlens; p.nseq = nseq;
  hipError_t e = attn::launch_fp8_prep(p, per_tensor != 0, (hipStream_t)hip_stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
