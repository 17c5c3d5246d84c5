// Decoding-shaped attention over key chunks (FlashDecoding, which the
// "FlashAttention-3" wiki page lists among the method's relatives; the
// online-softmax recurrence of "Flash Attention 3：让 GPU 跑满的注意力计算",
// §2.2, over one chunk of keys).
//
// With a few query rows per (batch, head) (decoding: one new token, or a few
// draft tokens) a tile of 32 query rows per MFMA would be mostly padding, and
// the work is a stream over K and V: 4 d bytes of 16-bit K/V per key against
// 4 d flops per query row, far below the matrix cores' balance point.  This
// kernel is shaped for that stream: no LDS ring and no MFMA.  Each lane
// loads an 8-element slice of a key row straight into registers (16 bytes of
// a 16-bit row, 8 bytes of an 8-bit cache row), a row takes d / 8 lanes and a
// wave d / 8-lane groups of keys, 512 / d keys per load.  The dot products
// run on the VALU in fp32, a DPP sum inside each lane group gives every lane
// of the group its key's score, and every lane keeps the online-softmax state
// (reference max, sum, 8 output columns) of the keys its group saw, with the
// lazy reference max of the prefill kernel.  A wave keeps two batches of
// loads in flight.  At the end the lane groups and the waves of the
// workgroup combine their states (the same rule the merge kernel applies
// across chunks) and the workgroup writes its chunk's normalised output and
// lse to the fp32 workspace, as the prefill kernel's key-chunk launches do.
//
// Work item: (batch, head, key chunk), all the head's query rows (at most
// kDecodeMaxRows).  Dense K/V ([B, H, Nk, d], causal masks with absolute
// indices, top-left) or an 8-bit paged cache (e4m3 or int8 codes with a
// per-(token, head) scale multiplying the score and the probability, as in
// the prefill kernel; the codes widen to fp32 exactly).  Over an 8-bit cache
// the queries may be e4m3 codes too, with one scale per (batch, head)
// (widened exactly, the scale applied in fp32).  A 16-bit paged cache
// stays on the prefill kernel's key-chunk launch, measured faster there
// (decode_shape).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_params.h"

namespace attn {
namespace {

constexpr int kDecWaves = 4;          // waves per workgroup
constexpr int kDecDepth = 2;          // steps per load batch (two batches in flight)
constexpr float kDecLazyBits = 4.0f;  // slack of the reference max (as the prefill kernel's)
constexpr int kKvDenseD = 0, kKvPagedD = 1, kKvE4m3D = 2, kKvInt8D = 3;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of G lanes (8, 16 or 32), in every lane of the
// group: exchanges within quads, then mirrors within half-rows and rows.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);   // quad: lanes 1 0 3 2
  v += dpp<0x4E>(v);   // quad: lanes 2 3 0 1
  v += dpp<0x141>(v);  // half-row mirror: sums of 8
  if constexpr (G >= 16) v += dpp<0x140>(v);  // row mirror: sums of 16
  if constexpr (G >= 32) v += __shfl_xor(v, 16);
  return v;
}

// Query tag: e4m3 codes with one fp32 scale per (batch, head), the tile
// scale of the fp8 layout [B, H, ceil(Nq / 128)] for Nq <= kDecodeMaxRows.
struct e4m3_query_t {};

// One lane's slice of a key or value row as loaded: 16 bytes of a 16-bit row,
// 8 bytes of codes.
template <int KV>
struct Raw {
  uint4 w;
};
template <>
struct Raw<kKvE4m3D> {
  uint2 w;
};
template <>
struct Raw<kKvInt8D> {
  uint2 w;
};

template <typename TT, int KV>
__device__ __forceinline__ void widen(const Raw<KV>& r, float (&f)[8]) {
  if constexpr (KV == kKvE4m3D) {
    const uint32_t ws[2] = {r.w.x, r.w.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], false);
      const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], true);
      f[4 * i + 0] = a[0];
      f[4 * i + 1] = a[1];
      f[4 * i + 2] = b[0];
      f[4 * i + 3] = b[1];
    }
  } else if constexpr (KV == kKvInt8D) {
    const uint32_t ws[2] = {r.w.x, r.w.y};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) f[4 * i + j] = (float)(int8_t)((ws[i] >> (8 * j)) & 0xff);
  } else {
    const uint32_t ws[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t a = unpack2(TT{}, ws[i]);
      f[2 * i] = a[0];
      f[2 * i + 1] = a[1];
    }
  }
}

template <typename TT, int D, int KV, int NQ, bool CAUSAL>
__global__ void __launch_bounds__(kDecWaves * 64) attn_decode_kernel(FwdParams p) {
  constexpr int LPK = D / 8;     // lanes per key row
  constexpr int KPL = 64 / LPK;  // keys per wave per step
  constexpr bool PAGED = KV != kKvDenseD;
  constexpr bool Q8 = KV == kKvE4m3D || KV == kKvInt8D;
  constexpr int ESZ = Q8 ? 1 : 2;  // bytes per cached element
  static_assert(!(PAGED && CAUSAL), "paged caches are read without a mask");
  __shared__ float red[kDecWaves][NQ][D + 2];

  const int w = blockIdx.x;
  const int hflat = w / p.n_split;  // b * H + h
  const int split = w - hflat * p.n_split;
  const int b = hflat / p.H, h = hflat - b * p.H;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int grp = lane / LPK, d0 = (lane % LPK) * 8;

  int nk = p.Nk;
  if constexpr (PAGED) nk = min(max(load_uniform(p.seqlens_k, b), 0), p.max_pages * p.page_size);
  const int kb = (int)min((int64_t)split * p.split_len, (int64_t)nk);
  const int ke = (int)min((int64_t)kb + p.split_len, (int64_t)nk);

  // query rows (scaled by c = scale log2 e: scores in base 2)
  float q[NQ][8];
#pragma unroll
  for (int r = 0; r < NQ; ++r) {
    if (r < p.Nq) {
      if constexpr (std::is_same_v<TT, e4m3_query_t>) {
        // codes widen exactly; the scale and c multiply in fp32
        Raw<kKvE4m3D> raw;
        raw.w = *(const uint2*)((const uint8_t*)p.q + ((int64_t)hflat * p.Nq + r) * D + d0);
        float f[8];
        widen<TT, kKvE4m3D>(raw, f);
        const float qs = load_uniform(p.q_scale, hflat) * p.c;
#pragma unroll
        for (int i = 0; i < 8; ++i) q[r][i] = f[i] * qs;
      } else {
        const uint4 raw = *(const uint4*)((const uint16_t*)p.q + ((int64_t)hflat * p.Nq + r) * D + d0);
        const uint32_t ws[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x2_t a = unpack2(TT{}, ws[i]);
          q[r][2 * i] = a[0] * p.c;
          q[r][2 * i + 1] = a[1] * p.c;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) q[r][i] = 0.f;
    }
  }
  float M[NQ], l[NQ], o[NQ][8];
#pragma unroll
  for (int r = 0; r < NQ; ++r) {
    M[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[r][i] = 0.f;
  }

  // step j of the workgroup covers keys kb + j KPL .. + KPL - 1; wave wv
  // takes steps wv, wv + kDecWaves, ...; lane group grp the key kb + j KPL +
  // grp.  Keys past ke re-read the chunk's last key (in bounds) and are
  // masked.
  const int n_steps = (ke - kb + KPL - 1) / KPL;
  auto row_of = [&](int j) -> int64_t {
    const int key = min(kb + j * KPL + grp, ke - 1);
    if constexpr (PAGED) {
      // the KPL keys of a step lie in one page (chunks and pages are whole
      // multiples of 64 keys): one table read per wave and step
      const int key0 = kb + j * KPL;
      const int pi = key0 / p.page_size;
      const int pg = min(max(load_uniform(p.block_table, (int64_t)b * p.max_pages + pi), 0), p.num_pages - 1);
      return ((int64_t)pg * p.page_size + (key - pi * p.page_size)) * p.H + h;
    } else {
      return (int64_t)hflat * p.Nk + key;
    }
  };
  struct Step {
    Raw<KV> k, v;
    float ks, vs;
  };
  auto load = [&](int j, Step& s) {
    const int64_t row = row_of(min(j, n_steps - 1));
    const uint8_t* kp = (const uint8_t*)p.k + (row * D + d0) * ESZ;
    const uint8_t* vp = (const uint8_t*)p.v + (row * D + d0) * ESZ;
    if constexpr (Q8) {
      s.k.w = *(const uint2*)kp;
      s.v.w = *(const uint2*)vp;
      s.ks = p.k_scale[row];
      s.vs = p.v_scale[row];
    } else {
      s.k.w = *(const uint4*)kp;
      s.v.w = *(const uint4*)vp;
      s.ks = 1.f;
      s.vs = 1.f;
    }
  };
  // the DEPTH steps of one batch: first every score (independent chains),
  // then one lazy reference-max check for the batch, then P and O
  auto process = [&](int j0, const Step (&S)[kDecDepth]) {
    float sc[kDecDepth][NQ];
#pragma unroll
    for (int u = 0; u < kDecDepth; ++u) {
      const int j = j0 + u * kDecWaves;
      const int key = kb + j * KPL + grp;
      const bool valid = j < n_steps && key < ke;
      float kf[8];
      widen<TT, KV>(S[u].k, kf);
#pragma unroll
      for (int r = 0; r < NQ; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(q[r][i], kf[i], acc);
        acc = group_sum<LPK>(acc);
        if constexpr (Q8) acc *= S[u].ks;
        const bool vis = valid && (!CAUSAL || key <= r);
        sc[u][r] = vis ? acc : -INFINITY;
      }
    }
    // lazy reference max: a lane moves its reference only when a score
    // passes it by more than kDecLazyBits (p <= 2^kDecLazyBits otherwise)
    float mb[NQ];
    bool up = false;
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
      mb[r] = sc[0][r];
#pragma unroll
      for (int u = 1; u < kDecDepth; ++u) mb[r] = fmaxf(mb[r], sc[u][r]);
      up |= mb[r] > M[r] + kDecLazyBits;
    }
    if (__any(up)) {
#pragma unroll
      for (int r = 0; r < NQ; ++r) {
        if (mb[r] > M[r] + kDecLazyBits) {
          const float mn = __builtin_ceilf(mb[r]);
          const float alpha = M[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[r] - mn);
          l[r] *= alpha;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[r][i] *= alpha;
          M[r] = mn;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kDecDepth; ++u) {
      float vf[8];
      widen<TT, KV>(S[u].v, vf);
#pragma unroll
      for (int r = 0; r < NQ; ++r) {
        const float pr = __builtin_amdgcn_exp2f(sc[u][r] - (M[r] == -INFINITY ? 0.f : M[r]));
        l[r] += pr;
        const float pv = Q8 ? pr * S[u].vs : pr;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[r][i] = __builtin_fmaf(pv, vf[i], o[r][i]);
      }
    }
  };

  if (n_steps > 0) {
    constexpr int SPAN = kDecWaves * kDecDepth;  // steps of one batch of every wave
    Step A[kDecDepth], Bn[kDecDepth];
#pragma unroll
    for (int u = 0; u < kDecDepth; ++u) load(wv + u * kDecWaves, A[u]);
    for (int j0 = wv; j0 < n_steps; j0 += 2 * SPAN) {
      // batch A (steps j0 ..) is in flight; issue batch B, then use A.  The
      // loads are unconditional (steps past the chunk re-read its last row):
      // behind a branch, the compiler would wait for every load at the join,
      // the batch just issued included.
      const int j1 = j0 + SPAN;
#pragma unroll
      for (int u = 0; u < kDecDepth; ++u) load(j1 + u * kDecWaves, Bn[u]);
      process(j0, A);
      if (j1 >= n_steps) break;
#pragma unroll
      for (int u = 0; u < kDecDepth; ++u) load(j1 + SPAN + u * kDecWaves, A[u]);
      process(j1, Bn);
    }
  }

  // combine the lane groups of the wave (offsets LPK .. 32), then the waves
#pragma unroll
  for (int r = 0; r < NQ; ++r) {
    float mw = M[r];
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
    const float f = M[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[r] - mw);
    float lw = l[r] * f;
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = o[r][i] * f;
#pragma unroll
      for (int off = LPK; off < 64; off <<= 1) x += __shfl_xor(x, off);
      o[r][i] = x;
    }
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wv][r][d0 + i] = o[r][i];
      if (lane == 0) {
        red[wv][r][D] = mw;
        red[wv][r][D + 1] = lw;
      }
    }
  }
  __syncthreads();
  // wave r % kDecWaves writes row r: lanes of group 0 hold its columns
  for (int r = wv; r < NQ && r < p.Nq; r += kDecWaves) {
    float mt = -INFINITY;
#pragma unroll
    for (int x = 0; x < kDecWaves; ++x) mt = fmaxf(mt, red[x][r][D]);
    float lt = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < kDecWaves; ++x) {
      const float mx = red[x][r][D];
      const float f = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - mt);
      lt += red[x][r][D + 1] * f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += red[x][r][d0 + i] * f;
    }
    if (grp == 0) {
      const int64_t prow = (int64_t)split * p.B * p.H * p.Nq + (int64_t)hflat * p.Nq + r;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      float* orow = p.o_part + prow * D + d0;
      *(float4*)orow = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      *(float4*)(orow + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
      if (lane == 0) p.lse_part[prow] = lt > 0.f ? (mt + __log2f(lt)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

template <typename TT, int D, int KV, bool CAUSAL>
hipError_t launch_decode_d(const FwdParams& p, hipStream_t st) {
  const int64_t n = (int64_t)p.n_split * p.B * p.H;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)n), block(kDecWaves * 64);
  static_assert(kDecodeMaxRows == 2, "one instantiation per row count");
  if (p.Nq <= 1) hipLaunchKernelGGL((attn_decode_kernel<TT, D, KV, 1, CAUSAL>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((attn_decode_kernel<TT, D, KV, 2, CAUSAL>), grid, block, 0, st, p);
  return hipGetLastError();
}

template <typename TT, int KV, bool CAUSAL>
hipError_t launch_decode_kv(int d, const FwdParams& p, hipStream_t st) {
  switch (d) {
    case 64: return launch_decode_d<TT, 64, KV, CAUSAL>(p, st);
    case 128: return launch_decode_d<TT, 128, KV, CAUSAL>(p, st);
    case 256: return launch_decode_d<TT, 256, KV, CAUSAL>(p, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename TT>
hipError_t launch_decode_t(int d, bool causal, int kv, const FwdParams& p, hipStream_t st) {
  switch (kv) {
    case kKvDenseD:
      return causal ? launch_decode_kv<TT, kKvDenseD, true>(d, p, st) : launch_decode_kv<TT, kKvDenseD, false>(d, p, st);
    case kKvE4m3D: return launch_decode_kv<TT, kKvE4m3D, false>(d, p, st);
    case kKvInt8D: return launch_decode_kv<TT, kKvInt8D, false>(d, p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_shape(int Nq, int kv) { return Nq <= kDecodeMaxRows && kv != kKvPagedD; }

hipError_t launch_decode(int dtype, int d, bool causal, int kv, const FwdParams& p, hipStream_t st) {
  if (!decode_shape(p.Nq, kv) || (causal && kv != kKvDenseD)) return hipErrorInvalidValue;
  if (dtype == 2) {
    // e4m3 queries: 8-bit paged caches only
    switch (kv) {
      case kKvE4m3D: return launch_decode_kv<e4m3_query_t, kKvE4m3D, false>(d, p, st);
      case kKvInt8D: return launch_decode_kv<e4m3_query_t, kKvInt8D, false>(d, p, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (dtype == 0) return launch_decode_t<f16_t>(d, causal, kv, p, st);
  return launch_decode_t<bf16_t>(d, causal, kv, p, st);
}

}  // namespace attn
