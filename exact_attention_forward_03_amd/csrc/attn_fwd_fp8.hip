// Exact-attention forward with e4m3 operands on gfx950 (CDNA4) fp8 MFMA.
//
// Inputs are the codes and per-128-row-tile scales written by the fp8
// pre-processing ("FlashAttention-3", "Three techniques" §3: FP8 products
// with block quantisation and incoherent processing); the softmax statistics
// stay in fp32 (the "two-stage softmax" of "Flash Attention 3：让 GPU 跑满的
// 注意力计算", §4.1.2: max and sum in higher precision, products in FP8).
// Output O is bfloat16, lse fp32.
//
// The kernel has the shape of the fp16/bf16 one (one workgroup per 32*NW
// query rows, K/V tiles double buffered in LDS, S^T = K Q^T so P stays in
// registers), with these differences:
//   * 32x32x64 e4m3 MFMA, fp32 accumulation; key tiles of 128 rows, so each
//     tile has exactly one K scale and one V scale;
//   * scores t = acc * (scale log2 e * s_q * s_k) in base 2; M = ceil(max t)
//     per row (an integer, so rescaling O and l is exact);
//   * P is rounded to e4m3 as e4m3(2^(t - M + 8) * w), w = s_v(tile) /
//     max_tiles s_v: the V tile's scale is folded into the exponent, so the
//     PV product needs no per-tile correction of O and the codes stay <= 256;
//     l sums the unrounded 2^(t - M) and O = (max s_v) 2^-8 sum P8 v8 / l;
//   * V is transposed byte-wise into LDS in the key order of P's registers.
#include "attn_device.h"
#include "attn_params.h"

namespace attn {
namespace {

constexpr int kFp8D = 128;
constexpr int kFp8BC = 128;
constexpr int kFp8NW = 8;
constexpr int kScaleRows = 128;

// Byte position of key k (0..127) inside a transposed V row: the PV MFMA
// takes 64 keys per step; lane half h, slot j of step g holds key
// 64 g + 32 (j / 16) + 8 ((j % 16) / 4) + 4 h + j % 4.
__device__ __forceinline__ int vt8_pos(int k) {
  const int g = k >> 6, kk = k & 63, blk = kk >> 5, k32 = kk & 31;
  const int h = (k32 >> 2) & 1;
  const int j = 16 * blk + 4 * (k32 >> 3) + (k32 & 3);
  return 64 * g + 32 * h + j;
}

// 4 rows x 4 bytes -> 4 columns x 4 bytes (byte transpose of a 4x4 block).
__device__ __forceinline__ void transpose4x4(const uint32_t r[4], uint32_t out[4]) {
  const uint32_t t01l = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
  const uint32_t t23l = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
  const uint32_t t01h = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
  const uint32_t t23h = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
}

__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <int NW, bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(2, 2)))
attn_fwd_fp8_kernel(FwdParams p) {
  constexpr int D = kFp8D, BC = kFp8BC;
  constexpr int BR = NW * 32, NT = NW * 64;
  constexpr int KP = D + 16;    // K row pitch in LDS (bytes)
  constexpr int VP = BC + 16;   // V^T row pitch in LDS (bytes)
  constexpr int KBUF = BC * KP, VBUF = D * VP;
  constexpr int KS = D / 64;    // MFMA k-steps of S^T
  constexpr int MB = BC / 32;   // 32-key blocks per tile
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  constexpr int PG = BC / 64;   // MFMA k-steps of O^T (64 keys each)
  constexpr int KCH = BC * D / 16 / NT;          // 16-byte K chunks per thread
  constexpr int VCH = (BC / 4) * (D / 4) / NT;   // 4x4-byte V blocks per thread
  static_assert(KCH * NT * 16 == BC * D && VCH * NT * 16 == BC * D, "tile split");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds8[];

  const int work = xcd_remap(blockIdx.x, p.n_work);
  const int head = work / p.tiles_per_head;
  const int t = work - head * p.tiles_per_head;
  const int qt = CAUSAL ? (p.tiles_per_head - 1 - t) : t;
  const int q_len = p.Nq, k_len = p.Nk;
  const int q0 = qt * BR;
  const int64_t q_row0 = (int64_t)head * p.Nq, k_row0 = (int64_t)head * p.Nk;
  const int nqs = (q_len + kScaleRows - 1) / kScaleRows;
  const int nks = (k_len + kScaleRows - 1) / kScaleRows;
  const float* __restrict__ sk = p.k_scale + (int64_t)head * nks;
  const float* __restrict__ sv = p.v_scale + (int64_t)head * nks;

  const uint8_t* __restrict__ Qp = (const uint8_t*)p.q + q_row0 * D;
  const uint8_t* __restrict__ Kp = (const uint8_t*)p.k + k_row0 * D;
  const uint8_t* __restrict__ Vp = (const uint8_t*)p.v + k_row0 * D;

  const int tid = threadIdx.x;
  const int wv = tid >> 6, lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int qw0 = q0 + wv * 32;
  const int my_q = qw0 + c;
  const bool q_ok = my_q < q_len;
  const bool wave_live = qw0 < q_len;

  // largest V scale of this head (every lane of every wave computes it)
  float sv_max = 0.f;
  for (int j = lane; j < nks; j += 64) sv_max = fmaxf(sv_max, sv[j]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) sv_max = fmaxf(sv_max, __shfl_xor(sv_max, s));
  const float lsv_max = sv_max > 0.f ? __log2f(sv_max) : 0.f;
  const float sq = wave_live ? p.q_scale[(int64_t)head * nqs + qw0 / kScaleRows] : 0.f;

  // Q fragments (B operand of S^T): row my_q, bytes [64 ks + 32 hh, +32)
  uint4 qf[KS][2];
  {
    const uint8_t* qrow = Qp + (int64_t)(q_ok ? my_q : 0) * D + 32 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks][0] = q_ok ? *(const uint4*)(qrow + 64 * ks) : zero4();
      qf[ks][1] = q_ok ? *(const uint4*)(qrow + 64 * ks + 16) : zero4();
    }
  }

  int n_kt = (k_len + BC - 1) / BC;
  if (CAUSAL) n_kt = min(n_kt, (min(q0 + BR, q_len) - 1) / BC + 1);
  int wave_kt = n_kt;
  if (!wave_live) wave_kt = 0;
  else if (CAUSAL) wave_kt = min(n_kt, (min(qw0 + 31, q_len - 1)) / BC + 1);

  uint8_t* const ldsK = lds8;
  uint8_t* const ldsV = lds8 + 2 * KBUF;
  uint4 kr[KCH];
  uint32_t vr[VCH][4];

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + i * NT;
      const int row = ch / (D / 16), col = (ch % (D / 16)) * 16;
      const int key = kt * BC + row;
      kr[i] = key < k_len ? *(const uint4*)(Kp + (int64_t)key * D + col) : zero4();
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int ch = tid + i * NT;
      const int kg = ch / (D / 4), dg = ch % (D / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kt * BC + 4 * kg + r;
        vr[i][r] = key < k_len ? *(const uint32_t*)(Vp + (int64_t)key * D + 4 * dg) : 0u;
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint8_t* kb = ldsK + buf * KBUF;
    uint8_t* vb = ldsV + buf * VBUF;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + i * NT;
      const int row = ch / (D / 16), col = (ch % (D / 16)) * 16;
      *(uint4*)(kb + row * KP + col) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int ch = tid + i * NT;
      const int kg = ch / (D / 4), dg = ch % (D / 4);
      uint32_t cols[4];
      transpose4x4(vr[i], cols);
      uint8_t* dst = vb + (4 * dg) * VP + vt8_pos(4 * kg);
#pragma unroll
      for (int j = 0; j < 4; ++j) *(uint32_t*)(dst + j * VP) = cols[j];
    }
  };

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  float M = -INFINITY, l = 0.f;
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) load_tile(kt + 1);

    if (kt < wave_kt) {
      const uint8_t* kb = ldsK + buf * KBUF;
      const uint8_t* vb = ldsV + buf * VBUF;
      const float cs = p.c * sq * sk[kt];
      const float svt = sv[kt];
      // log2 of 2^8 w: P codes are e4m3(2^(t - M) * 2^8 * s_v / max s_v)
      const float bias = 8.f + (svt > 0.f ? __log2f(svt) - lsv_max : -INFINITY);

      f32x16_t s[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        s[mb] = f32x16_t{};
        const uint8_t* krow = kb + (mb * 32 + c) * KP + 32 * hh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s[mb] = mfma32_fp8(*(const uint4*)(krow + 64 * ks), *(const uint4*)(krow + 64 * ks + 16), qf[ks][0],
                             qf[ks][1], s[mb]);
      }

      const int key0 = kt * BC;
      const bool need_mask = (key0 + BC > k_len) || (CAUSAL && key0 + BC - 1 > qw0);
      float tmax = -INFINITY;
      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + mb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            const bool ok = key < k_len && (!CAUSAL || key <= my_q);
            s[mb][i] = ok ? s[mb][i] * cs : -INFINITY;
            tmax = fmaxf(tmax, s[mb][i]);
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[mb][i]);
        tmax *= cs;  // scales are >= 0
      }
      tmax = max_halves(tmax);
      const float m_new = fmaxf(M, __builtin_ceilf(tmax));
      if (__any(m_new > M)) {
        const float alpha = (m_new == M) ? 1.f : __builtin_amdgcn_exp2f(M - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
      M = m_new;
      const float m_use = (M == -INFINITY) ? 0.f : M;
      const float off = bias - m_use;

      float rs = 0.f;
      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s[mb][i] = __builtin_amdgcn_exp2f(s[mb][i] + off);
            rs += s[mb][i];
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s[mb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][i], cs, off));
            rs += s[mb][i];
          }
      }
      // rs sums 2^(t - M) * 2^bias; l keeps the unweighted sum
      l += bias == -INFINITY ? 0.f : rs * __builtin_amdgcn_exp2f(-bias);

      // P codes: step g takes key blocks 2g (slots 0..15) and 2g+1 (slots 16..31)
#pragma unroll
      for (int g = 0; g < PG; ++g) {
        const f32x16_t& a = s[2 * g];
        const f32x16_t& b = s[2 * g + 1];
        const uint4 p0 = make_uint4(pack4_e4m3(a[0], a[1], a[2], a[3]), pack4_e4m3(a[4], a[5], a[6], a[7]),
                                    pack4_e4m3(a[8], a[9], a[10], a[11]), pack4_e4m3(a[12], a[13], a[14], a[15]));
        const uint4 p1 = make_uint4(pack4_e4m3(b[0], b[1], b[2], b[3]), pack4_e4m3(b[4], b[5], b[6], b[7]),
                                    pack4_e4m3(b[8], b[9], b[10], b[11]), pack4_e4m3(b[12], b[13], b[14], b[15]));
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint8_t* vrow = vb + (db * 32 + c) * VP + 64 * g + 32 * hh;
          oacc[db] = mfma32_fp8(*(const uint4*)vrow, *(const uint4*)(vrow + 16), p0, p1, oacc[db]);
        }
      }
    }

    if (kt + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = sum_halves(l);
  if (q_ok) {
    const float f = l_tot > 0.f ? sv_max * (1.f / 256.f) / l_tot : 0.f;
    uint16_t* orow = (uint16_t*)p.o + (q_row0 + my_q) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dcol = db * 32 + 8 * g + 4 * hh;
        *(uint2*)(orow + dcol) = make_uint2(pack2(bf16_t{}, oacc[db][4 * g + 0] * f, oacc[db][4 * g + 1] * f),
                                            pack2(bf16_t{}, oacc[db][4 * g + 2] * f, oacc[db][4 * g + 3] * f));
      }
    if (hh == 0) p.lse[q_row0 + my_q] = l_tot > 0.f ? (M + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int NW, bool CAUSAL>
hipError_t launch_fp8(const FwdParams& p, hipStream_t st) {
  constexpr int lds = 2 * (kFp8BC * (kFp8D + 16) + kFp8D * (kFp8BC + 16));
  auto kern = attn_fwd_fp8_kernel<NW, CAUSAL>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(p.n_work), dim3(NW * 64), lds, st, p);
  return hipGetLastError();
}

}  // namespace

int fwd_fp8_block_rows() { return 32 * kFp8NW; }

hipError_t launch_fwd_fp8(int d, bool causal, const FwdParams& p, hipStream_t st) {
  if (d != kFp8D) return hipErrorInvalidValue;
  return causal ? launch_fp8<kFp8NW, true>(p, st) : launch_fp8<kFp8NW, false>(p, st);
}

}  // namespace attn
