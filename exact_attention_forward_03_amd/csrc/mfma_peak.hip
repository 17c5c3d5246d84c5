// MFMA throughput probe for the measurement harness (libattn_probe.so, not
// part of the attention C ABI): the dense matrix-core rate this GPU sustains
// on a stream of independent 32x32 MFMAs with operands in registers, which
// the attention kernels' rate is compared with next to the spec peak.
//
//   int attn_probe_mfma_tflops(int kind, double* tflops, void* hip_stream)
//     kind 0: v_mfma_f32_32x32x16_bf16; kind 1: v_mfma_f32_32x32x64 e4m3.
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

__global__ void __launch_bounds__(256) mfma_bf16_probe(float* out, float seed) {
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
    b[i] = (__bf16)(seed * (float)i);
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < kIters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) mfma_fp8_probe(float* out, int seed) {
  i32x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)(0x38383838u ^ (uint32_t)(seed * (threadIdx.x + i)) & 0x07070707u);
    b[i] = (int)(0x38383838u ^ (uint32_t)(seed * i) & 0x07070707u);
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < kIters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" int attn_probe_mfma_tflops(int kind, double* tflops, void* hip_stream) {
  if (!tflops || (kind != 0 && kind != 1)) return -1;
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
      if (kind == 0) hipLaunchKernelGGL(mfma_bf16_probe, dim3(blocks), dim3(256), 0, st, out, 1e-3f);
      else hipLaunchKernelGGL(mfma_fp8_probe, dim3(blocks), dim3(256), 0, st, out, 7);
      if (hipGetLastError() != hipSuccess || hipEventRecord(e1, st) != hipSuccess ||
          hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
        rc = -3;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(out);
  if (rc != 0 || ms <= 0.f) return rc != 0 ? rc : -3;
  const double flops_per_mfma = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  const double mfmas = (double)blocks * 4 /* waves */ * kIters * 4;
  *tflops = mfmas * flops_per_mfma / (ms * 1e-3) / 1e12;
  return 0;
}
