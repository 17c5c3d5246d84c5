// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, MFMA wrappers, packing, cross-lane exchange and the
// XCD-aware workgroup remapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct f16_t {};   // tag: IEEE binary16 storage
struct bf16_t {};  // tag: bfloat16 storage

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// 32x32 MFMA with K = 16 (fp16/bf16) and K = 64 (e4m3), fp32 accumulation.
//
// Operand layout (both A [32 x K] and B [K x 32]): lane l holds row/column
// (l % 32) and the contiguous K-slice of its half (l / 32).  The 16 fp32
// results of lane l are column n = l % 32, rows 8*(i/4) + 4*(l/32) + i%4.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16_t mfma32(f16_t, const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                               __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(bf16_t, const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// e4m3 x e4m3: each operand is 32 bytes per lane (two uint4).  The zero scale
// selectors select the unscaled instruction.
__device__ __forceinline__ f32x16_t mfma32_fp8(const uint4& a0, const uint4& a1, const uint4& b0,
                                               const uint4& b1, const f32x16_t& c) {
  i32x8_t a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  i32x8_t b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Two fp32 values -> one dword of two 16-bit floats (round to nearest even).
__device__ __forceinline__ uint32_t pack2(f16_t, float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
}
__device__ __forceinline__ uint32_t pack2(bf16_t, float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// The two values of a packed pair of 16-bit floats, widened to fp32.
__device__ __forceinline__ f32x2_t unpack2(f16_t, uint32_t pk) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2_t, pk), f32x2_t);
}
__device__ __forceinline__ f32x2_t unpack2(bf16_t, uint32_t pk) {
  return (f32x2_t){__builtin_bit_cast(float, pk << 16), __builtin_bit_cast(float, pk & 0xffff0000u)};
}
// Residual of a rounded pair: pack2(a - round(a), b - round(b)), given pk = pack2(a, b).
// a - round(a) is exact in fp32.
template <typename TT>
__device__ __forceinline__ uint32_t residual2(TT t, uint32_t pk, float a, float b) {
  const f32x2_t r = unpack2(t, pk);
  return pack2(t, a - r[0], b - r[1]);
}

// Reductions across the two halves of the wave (lane l and lane l ^ 32, the
// two halves of a 32x32 MFMA column) with v_permlane32_swap, which exchanges
// the upper 32 lanes of its first register with the lower 32 lanes of its
// second: with both holding x, the first ends up with the lower half of x in
// all 64 lanes and the second with the upper half.  The instruction is
// written as inline asm because the compiler builtin loses its second result
// (it returns the first one twice).  The s_nop pairs keep two wait states
// between the swap and the VALU writes of its operands on either side.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_halves(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_halves(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}

// Workgroups are dealt to the 8 XCDs round-robin (id % 8).  Remap the
// hardware id so that consecutive work items land on the same XCD and share
// its L2: work = offset(xcd) + id / 8, a bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = id & 7, slot = id >> 3;
  return x * per + (x < rem ? x : rem) + slot;
}

// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no
// swizzle, no stride; num_records counts bytes.
constexpr int kBufferFlags = 0x00020000;

// A wave-uniform int32 read through the scalar data cache (s_load): it does
// not count against the vector-memory counter that paces the tile loads.
__device__ __forceinline__ int load_uniform(const int32_t* ptr, int64_t idx) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(idx & 0xffffffff));
  const int hi = __builtin_amdgcn_readfirstlane((int)(idx >> 32));
  const int64_t i = ((int64_t)hi << 32) | (uint32_t)lo;
  return ((const __attribute__((address_space(4))) int32_t*)ptr)[i];
}
__device__ __forceinline__ float load_uniform(const float* ptr, int64_t idx) {
  return __builtin_bit_cast(float, load_uniform((const int32_t*)ptr, idx));
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// f(kw, vw, kr, vr) with four LDS ring buffers passed as restrict pointers;
// the caller guarantees that they do not overlap.  A step that fills two
// buffers with direct-to-LDS loads (kw, vw) and reads two others (kr, vr)
// runs its body through this, so that the compiler knows the reads do not
// depend on those loads and does not wait for them before the first read.
template <typename F>
__device__ __forceinline__ void with_disjoint(uint8_t* __restrict__ kw, uint8_t* __restrict__ vw,
                                              const uint8_t* __restrict__ kr, const uint8_t* __restrict__ vr, F&& f) {
  f(kw, vw, kr, vr);
}

// f(w, r) with an LDS buffer that direct-to-LDS loads fill (w) and one that
// the step reads (r) passed as restrict pointers; the caller guarantees they
// do not overlap (the two-pointer form of with_disjoint).
template <typename F>
__device__ __forceinline__ void with_slots(uint8_t* __restrict__ w, const uint8_t* __restrict__ r, F&& f) {
  f(w, r);
}

}  // namespace attn
