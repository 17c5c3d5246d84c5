// FP8 pre-processing of one tensor x [B*H, N, d]: incoherent processing
// (random sign flip and Hadamard rotation along d) and block quantisation to
// e4m3 with one fp32 scale per 128-row tile ("FlashAttention-3", "Three
// techniques" §3: block quantisation; incoherent processing Q' = QM, K' = KM
// with M a Hadamard matrix times random +-1, applied before quantising).
//
// One workgroup (4 d threads) per (b*h, 128-row tile); the whole tile stays
// in registers, so x is read once and the codes are written once.  A row of d
// values is spread over d/8 lanes, 8 consecutive values per lane.  The
// Hadamard transform H_d (Sylvester order) is a product of one butterfly
// (a, b) -> (a + b, a - b) per bit of the column index: the three low bits are
// done inside the lane, the others between lanes (lane ^ 1, ^ 2, ...).
// Then the tile's amax, s = amax / 448 (1 if the tile is all zero; at least
// 2^-149, the smallest positive fp32, where amax / 448 would underflow), and
// code = e4m3(x' / s): x' / s correctly rounded to fp32, then rounded to
// nearest even e4m3.
//
// A variable-length batch ([H, T, d] with cu_seqlens) restarts the tiles at
// every sequence, so no tile (and no scale) spans two sequences.
//
// Per-tensor mode runs three launches: the tile amaxes into the scale array,
// one workgroup turning their maximum into s for every entry, and the
// quantisation with that s.
#include "attn_device.h"
#include "attn_params.h"
#include "attn_sched.h"

namespace attn {
namespace {

constexpr int kPrepThreads = 256;  // the tensor-scale pass
// Quantisation workgroups: 4 d threads, so each thread holds four row pieces
// of 8 values (measured fastest for d = 64, 128 and 256; fewer, larger
// pieces per thread left the last round of workgroups half empty).
template <int D>
constexpr int kTileThreads = 4 * D;
constexpr int kTileRows = 128;
constexpr float kE4m3Max = 448.0f;
// Smallest positive fp32: the scale of a tile whose amax / 448 underflows
// (amax < 448 * 2^-149), so its codes x / s stay finite (and exact).
constexpr float kF32Tiny = 0x1p-149f;

__device__ __forceinline__ void load8(const float* src, float v[8]) {
  const float4 a = *(const float4*)src, b = *(const float4*)(src + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* src, float v[8], bf16_t) {
  const uint4 a = *(const uint4*)src;
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const uint16_t* src, float v[8], f16_t) {
  const uint4 a = *(const uint4*)src;
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2_t f = __builtin_convertvector(__builtin_bit_cast(f16x2_t, w[i]), f32x2_t);
    v[2 * i] = f[0];
    v[2 * i + 1] = f[1];
  }
}

// v from lane (lane ^ S) with S < 16, by DPP lane permutes inside 16-lane
// rows (VALU only): XOR 1 and XOR 2 are quad permutations; the half-row
// mirror maps lane i to i ^ 7 and the row mirror to i ^ 15, so XOR 4 =
// mirror-half then XOR 3, and XOR 8 = mirror then mirror-half.  Larger
// strides go through ds_bpermute.
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppQuadXor3 = 0x1B;
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141;
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int S>
__device__ __forceinline__ float xor_lanes(float v) {
  if constexpr (S == 1) return dpp<kDppQuadXor1>(v);
  else if constexpr (S == 2) return dpp<kDppQuadXor2>(v);
  else if constexpr (S == 4) return dpp<kDppQuadXor3>(dpp<kDppRowHalfMirror>(v));
  else if constexpr (S == 8) return dpp<kDppRowHalfMirror>(dpp<kDppRowMirror>(v));
  else return __shfl_xor(v, S);
}

// Four fp32 values -> four e4m3 codes in one dword (round to nearest even).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// One butterfly stage between lanes cl and cl ^ S (no-op when S >= L).
template <int S, int L>
__device__ __forceinline__ void lane_stage(float (&v)[8], int cl) {
  if constexpr (S < L) {
    const float sg = (cl & S) ? -1.f : 1.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float o = xor_lanes<S>(v[j]);
      v[j] = __builtin_fmaf(sg, v[j], o);  // lower: o + v, upper: o - v (exact: a sign flip)
    }
  }
}

// Maximum over a workgroup of NT threads (red: NT / 64 floats of LDS).
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s));
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = fmaxf(m, red[i]);
  return m;
}

// MODE 0: block scales; 1: write the tile amax only; 2: quantise with the
// scale already stored for the tile (per-tensor).
template <int IN, int D, int MODE>
__global__ void __launch_bounds__(kTileThreads<D>) fp8_prep_kernel(PrepParams p) {
  constexpr int NT = kTileThreads<D>;
  constexpr int L = D / 8;                // lanes per row
  constexpr int RPP = NT / L;             // rows per pass
  constexpr int PASSES = kTileRows / RPP;
  __shared__ float red[NT / 64];

  const int nt = (p.N + kTileRows - 1) / kTileRows + (p.cu ? p.nseq : 0);  // scale entries per head
  const int bh = blockIdx.x / nt;
  const int tile = blockIdx.x - bh * nt;
  const int tid = threadIdx.x;
  const int rl = tid / L, cl = tid % L;
  const int64_t base = (int64_t)bh * p.N;
  // rows [row0, row_end) of this tile; a variable-length batch restarts the
  // tiles at every sequence, tile j of sequence s at entry
  // floor(cu[s] / 128) + s + j (sched::slot_tile; prefix sums clamped into
  // [0, N])
  int row0 = tile * kTileRows, row_end = p.N;
  if (p.cu) {
    sched::SlotTile st;
    if (!sched::slot_tile<kTileRows>(p.cu, p.nseq, p.N, p.cu, p.N, tile, st)) {
      // an entry no tile owns: 1 (block scales), 0 (tile amax, so it does
      // not raise the tensor amax); the tensor-scale pass then overwrites it
      if (MODE != 2 && tid == 0) p.scale[bh * nt + tile] = MODE == 1 ? 0.f : 1.f;
      return;
    }
    row0 = st.a + st.j * kTileRows;
    row_end = st.e;
  }

  float sg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sg[j] = p.signs ? p.signs[cl * 8 + j] : 1.f;
  const float norm = p.signs ? 1.0f / __builtin_sqrtf((float)D) : 1.0f;

  float v[PASSES][8];
  float amax = 0.f;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int row = row0 + ps * RPP + rl;
    if (row < row_end) {
      const int64_t off = (base + row) * D + cl * 8;
      if constexpr (IN == 3) load8((const float*)p.x + off, v[ps]);
      else if constexpr (IN == 1) load8((const uint16_t*)p.x + off, v[ps], bf16_t{});
      else load8((const uint16_t*)p.x + off, v[ps], f16_t{});
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[ps][j] = 0.f;
    }
    if (p.signs) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[ps][j] *= sg[j];
      // butterflies on the three in-lane bits of the column index
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!(j & h)) {
            const float a = v[ps][j], b = v[ps][j + h];
            v[ps][j] = a + b;
            v[ps][j + h] = a - b;
          }
      // butterflies on the lane bits: the lower partner keeps a + b, the upper a - b
      lane_stage<1, L>(v[ps], cl);
      lane_stage<2, L>(v[ps], cl);
      lane_stage<4, L>(v[ps], cl);
      lane_stage<8, L>(v[ps], cl);
      lane_stage<16, L>(v[ps], cl);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[ps][j] *= norm;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[ps][j]));
  }

  const int sidx = bh * nt + tile;
  float s;
  if constexpr (MODE == 2) {
    s = p.scale[sidx];
  } else {
    const float tmax = block_max<NT>(amax, red);
    if constexpr (MODE == 1) {
      if (tid == 0) p.scale[sidx] = tmax;
      return;
    }
    s = tmax > 0.f ? fmaxf(tmax / kE4m3Max, kF32Tiny) : 1.0f;
    if (tid == 0) p.scale[sidx] = s;
  }

  // x / s correctly rounded, by Markstein's division: with y = RN(1/s) (one
  // IEEE division per thread), q = RN(x y), r = x - q s (exact with an fma)
  // and RN(q + r y) = RN(x / s).  Tiles with a tiny scale, where r could
  // underflow, use the IEEE division itself.
  const float y = 1.0f / s;
  const bool markstein = s >= 0x1p-80f;
  auto quot = [&](float x) {
    const float q = x * y;
    return __builtin_fmaf(__builtin_fmaf(-q, s, x), y, q);
  };
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int row = row0 + ps * RPP + rl;
    if (row < row_end) {
      float z[8];
      if (markstein) {
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = quot(v[ps][j]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = v[ps][j] / s;
      }
      const uint2 w = make_uint2(pack4_e4m3(z[0], z[1], z[2], z[3]), pack4_e4m3(z[4], z[5], z[6], z[7]));
      *(uint2*)(p.x8 + (base + row) * D + cl * 8) = w;
    }
  }
}

// Per-tensor: every entry of the scale array becomes max(entries) / 448.
__global__ void __launch_bounds__(kPrepThreads) tensor_scale_kernel(float* scale, int n) {
  __shared__ float red[kPrepThreads / 64];
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += kPrepThreads) m = fmaxf(m, scale[i]);
  m = block_max<kPrepThreads>(m, red);
  const float s = m > 0.f ? fmaxf(m / kE4m3Max, kF32Tiny) : 1.0f;
  for (int i = threadIdx.x; i < n; i += kPrepThreads) scale[i] = s;
}

template <int IN, int D>
hipError_t launch_in_d(const PrepParams& p, bool per_tensor, hipStream_t st) {
  const int nt = (p.N + kTileRows - 1) / kTileRows + (p.cu ? p.nseq : 0);
  const int64_t grid = (int64_t)nt * p.BH;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (!per_tensor) {
    hipLaunchKernelGGL((fp8_prep_kernel<IN, D, 0>), dim3((unsigned)grid), dim3(kTileThreads<D>), 0, st, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fp8_prep_kernel<IN, D, 1>), dim3((unsigned)grid), dim3(kTileThreads<D>), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(kPrepThreads), 0, st, p.scale, (int)grid);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fp8_prep_kernel<IN, D, 2>), dim3((unsigned)grid), dim3(kTileThreads<D>), 0, st, p);
  return hipGetLastError();
}

template <int IN>
hipError_t launch_in(const PrepParams& p, bool per_tensor, hipStream_t st) {
  switch (p.d) {
    case 64: return launch_in_d<IN, 64>(p, per_tensor, st);
    case 128: return launch_in_d<IN, 128>(p, per_tensor, st);
    case 256: return launch_in_d<IN, 256>(p, per_tensor, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fp8_prep(const PrepParams& p, bool per_tensor, hipStream_t st) {
  switch (p.x_dtype) {
    case 3: return launch_in<3>(p, per_tensor, st);
    case 1: return launch_in<1>(p, per_tensor, st);
    case 0: return launch_in<0>(p, per_tensor, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
