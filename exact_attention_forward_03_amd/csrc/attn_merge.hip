// Merge of attention results computed over disjoint key chunks (the online
// softmax combination of "Flash Attention 3：让 GPU 跑满的注意力计算", §2.2,
// applied to any number of blocks; FlashDecoding in the related work of the
// "FlashAttention-3" wiki page):
//
//     lse = ln sum_s e^{lse_s},    O = sum_s e^{lse_s - lse} O_s.
//
// The partial outputs O_s are normalised fp32 rows; a chunk that saw no key
// has lse_s = -inf and contributes nothing; a row with no key at all gives
// O = 0, lse = -inf.  Memory-bound: each thread owns four columns of one row,
// reads the S partial values of its row (the largest lse_s first, so that no
// exponential overflows) and writes four fp16/bf16 values.
#include "attn_device.h"
#include "attn_params.h"

namespace attn {
namespace {

constexpr int kMergeThreads = 256;

template <typename TT, int D>
__global__ void __launch_bounds__(kMergeThreads) attn_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;                 // threads per row
  constexpr int RPB = kMergeThreads / TPR;   // rows per workgroup
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int col = (threadIdx.x % TPR) * 4;
  if (row >= p.rows) return;

  float m = -INFINITY;
  for (int s = 0; s < p.S; ++s) m = fmaxf(m, p.lse_part[(int64_t)s * p.rows + row]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < p.S; ++s) {
      const float ls = p.lse_part[(int64_t)s * p.rows + row];
      if (ls == -INFINITY) continue;
      const float w = expf(ls - m);
      const float4 o = *(const float4*)(p.o_part + ((int64_t)s * p.rows + row) * D + col);
      acc.x = __builtin_fmaf(w, o.x, acc.x);
      acc.y = __builtin_fmaf(w, o.y, acc.y);
      acc.z = __builtin_fmaf(w, o.z, acc.z);
      acc.w = __builtin_fmaf(w, o.w, acc.w);
      tot += w;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  uint16_t* orow = (uint16_t*)p.o + row * D + col;
  *(uint2*)orow = make_uint2(pack2(TT{}, acc.x * inv, acc.y * inv), pack2(TT{}, acc.z * inv, acc.w * inv));
  if (col == 0) p.lse[row] = tot > 0.f ? m + logf(tot) : -INFINITY;
}

template <typename TT>
hipError_t launch_merge_t(const MergeParams& p, hipStream_t st) {
  auto grid = [&](int d) { return (unsigned)((p.rows + (kMergeThreads / (d / 4)) - 1) / (kMergeThreads / (d / 4))); };
  switch (p.d) {
    case 64: hipLaunchKernelGGL((attn_merge_kernel<TT, 64>), dim3(grid(64)), dim3(kMergeThreads), 0, st, p); break;
    case 128: hipLaunchKernelGGL((attn_merge_kernel<TT, 128>), dim3(grid(128)), dim3(kMergeThreads), 0, st, p); break;
    case 256: hipLaunchKernelGGL((attn_merge_kernel<TT, 256>), dim3(grid(256)), dim3(kMergeThreads), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  if (p.rows / 4 > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  return p.o_dtype == 0 ? launch_merge_t<f16_t>(p, st) : launch_merge_t<bf16_t>(p, st);
}

}  // namespace attn
