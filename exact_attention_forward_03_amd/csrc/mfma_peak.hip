// MFMA throughput probe for the measurement harness (libattn_probe.so, not
// part of the attention C ABI): the dense matrix-core rate this GPU sustains
// on a stream of independent 32x32 MFMAs with operands in registers, which
// the attention kernels' rate is compared with next to the spec peak.
//
//   int attn_probe_mfma_tflops(int kind, double* tflops, void* hip_stream)
//     kind 0: v_mfma_f32_32x32x16_bf16; kind 1: v_mfma_f32_32x32x64 e4m3;
//     kinds 2 and 3: the same on random operand bits (each MFMA of a chain
//     takes its own pair of operand registers, filled from a counter hash:
//     bf16 of N(0,1)-like magnitude, e4m3 codes without NaN).  The chip
//     lowers its clock under the power of switching operand bits, so kinds
//     2 and 3 give the rate attention's data can reach; kinds 0 and 1
//     (constant operands) the rate of the matrix cores at a higher clock.
//     Launches 2 workgroups of 4 waves per CU (two waves per SIMD), each wave
//     issuing 4 independent accumulator chains, times the launch with HIP
//     events and synchronises the host.  Returns 0, or -1 on a bad argument,
//     -3 on a HIP error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kIters = 2048;  // 4 MFMAs each

// 32 pseudo-random bits from (a, b): a small counter hash (splitmix-style
// finaliser), enough to make operand bits switch like real data.
__device__ __forceinline__ uint32_t probe_hash(uint32_t a, uint32_t b) {
  uint32_t x = a * 0x9E3779B9u ^ (b + 0x7F4A7C15u);
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return x;
}

// bf16 of N(0,1)-like magnitude from 16 random bits: sign, exponent
// 120..127 (magnitudes 2^-7 .. 1.99), 7 random mantissa bits
__device__ __forceinline__ uint32_t probe_bf16_pair(uint32_t h) {
  const uint32_t lo = (h & 0x807fu) | ((120u + ((h >> 8) & 7u)) << 7);
  const uint32_t g = (h >> 16) | (h << 16);
  const uint32_t hi = (g & 0x807fu) | ((120u + ((g >> 8) & 7u)) << 7);
  return lo | (hi << 16);
}

template <bool RANDOM>
__global__ void __launch_bounds__(256) mfma_bf16_probe(float* out, float seed) {
  constexpr int R = RANDOM ? 8 : 1;  // operand register sets
  bf16x8_t a[R], b[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (RANDOM) {
      uint32_t wa[4], wb[4];
      for (int i = 0; i < 4; ++i) {
        wa[i] = probe_bf16_pair(probe_hash(blockIdx.x * 256 + threadIdx.x, r * 16 + i));
        wb[i] = probe_bf16_pair(probe_hash(blockIdx.x * 256 + threadIdx.x, r * 16 + 8 + i));
      }
      a[r] = __builtin_bit_cast(bf16x8_t, make_uint4(wa[0], wa[1], wa[2], wa[3]));
      b[r] = __builtin_bit_cast(bf16x8_t, make_uint4(wb[0], wb[1], wb[2], wb[3]));
    } else {
      for (int i = 0; i < 8; ++i) {
        a[r][i] = (__bf16)(seed * (float)(threadIdx.x + i));
        b[r][i] = (__bf16)(seed * (float)i);
      }
    }
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < kIters; it += R / 4 > 0 ? R / 4 : 1) {
#pragma unroll
    for (int r = 0; r < (R >= 4 ? R : 4); r += 4) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + 0) % R], b[(r + 0) % R], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + 1) % R], b[(r + 1) % R], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + 2) % R], b[(r + 2) % R], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + 3) % R], b[(r + 3) % R], c3, 0, 0, 0);
    }
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <bool RANDOM>
__global__ void __launch_bounds__(256) mfma_fp8_probe(float* out, int seed) {
  constexpr int R = RANDOM ? 8 : 1;
  i32x8_t a[R], b[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    for (int i = 0; i < 8; ++i) {
      if (RANDOM) {
        // e4m3 codes with bit 3 clear: never 0x7f / 0xff (NaN)
        a[r][i] = (int)(probe_hash(blockIdx.x * 256 + threadIdx.x, r * 16 + i) & 0xF7F7F7F7u);
        b[r][i] = (int)(probe_hash(blockIdx.x * 256 + threadIdx.x, r * 16 + 8 + i) & 0xF7F7F7F7u);
      } else {
        a[r][i] = (int)(0x38383838u ^ (uint32_t)(seed * (threadIdx.x + i)) & 0x07070707u);
        b[r][i] = (int)(0x38383838u ^ (uint32_t)(seed * i) & 0x07070707u);
      }
    }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < kIters; it += R / 4 > 0 ? R / 4 : 1) {
#pragma unroll
    for (int r = 0; r < (R >= 4 ? R : 4); r += 4) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(r + 0) % R], b[(r + 0) % R], c0, 0, 0, 0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(r + 1) % R], b[(r + 1) % R], c1, 0, 0, 0, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(r + 2) % R], b[(r + 2) % R], c2, 0, 0, 0, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(r + 3) % R], b[(r + 3) % R], c3, 0, 0, 0, 0, 0, 0);
    }
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" int attn_probe_mfma_tflops(int kind, double* tflops, void* hip_stream) {
  if (!tflops || kind < 0 || kind > 3) return -1;
  hipStream_t st = (hipStream_t)hip_stream;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return -3;
  const int blocks = 2 * prop.multiProcessorCount;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return -3;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 0;
  float ms = 0.f;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    rc = -3;
  } else {
    for (int rep = 0; rep < 2 && rc == 0; ++rep) {  // the first launch warms up
      if (hipEventRecord(e0, st) != hipSuccess) rc = -3;
      switch (kind) {
        case 0: hipLaunchKernelGGL(mfma_bf16_probe<false>, dim3(blocks), dim3(256), 0, st, out, 1e-3f); break;
        case 1: hipLaunchKernelGGL(mfma_fp8_probe<false>, dim3(blocks), dim3(256), 0, st, out, 7); break;
        case 2: hipLaunchKernelGGL(mfma_bf16_probe<true>, dim3(blocks), dim3(256), 0, st, out, 1e-3f); break;
        default: hipLaunchKernelGGL(mfma_fp8_probe<true>, dim3(blocks), dim3(256), 0, st, out, 7); break;
      }
      if (hipGetLastError() != hipSuccess || hipEventRecord(e1, st) != hipSuccess ||
          hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
        rc = -3;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(out);
  if (rc != 0 || ms <= 0.f) return rc != 0 ? rc : -3;
  const double flops_per_mfma = (kind % 2 == 0) ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  const double mfmas = (double)blocks * 4 /* waves */ * kIters * 4;
  *tflops = mfmas * flops_per_mfma / (ms * 1e-3) / 1e12;
  return 0;
}
