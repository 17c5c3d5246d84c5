// Exact attention forward for fp16/bf16 on gfx950 (CDNA4).
//
// One workgroup owns a block of BR = 32*NW query rows of one (batch, head)
// — or one (sequence, head) of a variable-length batch — and streams the
// keys and values through LDS in tiles of BC rows, keeping the online-softmax
// state in registers ("Flash Attention 3：让 GPU 跑满的注意力计算", §2.1 tiling,
// §2.2 online softmax, §3.1 one independent query block per workgroup).
//
// Per wave (32 query rows, 64 lanes):
//   * S^T = K Q^T on 32x32x16 MFMA: K rows are the A operand (read from LDS),
//     the wave's Q rows are the B operand (held in registers for the whole
//     kernel).  In the result every lane owns ONE query (lane % 32) and 16
//     keys per 32-key block, so the row max/sum are in-register reductions
//     plus one exchange between the two wave halves (v_permlane32_swap).
//   * The probabilities P^T come out of the MFMA already in the B-operand
//     layout of the second product, O^T = V^T P^T: they are converted to
//     fp16/bf16 in registers and never touch LDS.
//   * V is written into LDS transposed ([d][key]), with keys permuted inside
//     each 16-key group so that one 16-byte LDS read gives a lane exactly
//     the 8 keys its P^T fragment holds.
//   * K/V tiles are double buffered: the global loads of tile j+1 are issued
//     before tile j is computed and land in LDS after it, with one barrier
//     per tile.
//
// Softmax in base 2 with an integer reference maximum.  For each row the
// kernel keeps M = ceil(max of the scores seen so far, times scale*log2 e),
// p = 2^(S*scale*log2e - M) <= 1, l = sum p (fp32, unrounded), and
// O = sum p v.  M only moves when a tile raises the row max past the current
// integer; then O and l are multiplied by 2^(M_old - M_new), an exact power
// of two.  Skipping that rescale whenever no row of the wave moved is what
// keeps the fp32 vector work per tile small.  The result O / l and
// lse = (M + log2 l) ln 2 equal the page's recurrence (which rescales by
// e^{m_old - m_new} at every tile) up to rounding; the reference point of
// the exponentials does not change the sum they define.
//
// P enters the second product rounded to fp16/bf16.  While some row of the
// wave has little weight accumulated (its mass sits on a few keys, so |O| can
// be as large as |V|), the rounding residual p - round(p) is multiplied in by
// a second MFMA pass, which makes the weights exact to ~16 more bits.

// Causal masking is top-left (key j visible to query i iff j <= i).  Key
// tiles entirely above a wave's diagonal are skipped by that wave; tiles
// entirely above the workgroup's diagonal are never loaded.  Only tiles that
// cross the diagonal or the end of the keys apply an element mask.
//
// Workgroup order: the hardware id is remapped so that consecutive work items
// — the query tiles of one head — run on the same XCD and share its L2 copy
// of that head's K and V; causal query tiles run heaviest first.

#include "attn_device.h"
#include "attn_params.h"

namespace attn {
namespace {

// Position of key k (within a tile) in a transposed V row: bits 2 and 3 of
// the index inside its 16-key group are swapped, so that keys
// {0-3, 8-11} (lanes 0..31) and {4-7, 12-15} (lanes 32..63) are contiguous.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3);
}

__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {  // [a.lo, b.lo]
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {  // [a.hi, b.hi]
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// A lane's partial row sum below this (in units of the row's reference
// maximum, i.e. fewer than ~16 effective keys for the whole row) switches on
// the residual product for P.
constexpr float kSplitBelow = 8.0f;

template <int D, int BC, int NW>
struct TileCfg {
  static constexpr int BR = NW * 32;        // query rows per workgroup
  static constexpr int NT = NW * 64;        // threads
  static constexpr int KP = D + 8;          // K row pitch in LDS (elements)
  static constexpr int VP = BC + 8;         // V^T row pitch in LDS (elements)
  static constexpr int KS = D / 16;         // MFMA k-steps of S^T = K Q^T
  static constexpr int MB = BC / 32;        // 32-key blocks per tile
  static constexpr int DB = D / 32;         // 32-row blocks of O^T
  static constexpr int KBUF = BC * KP;      // elements of one K buffer
  static constexpr int VBUF = D * VP;       // elements of one V^T buffer
  static constexpr int KCH = BC * D / 8 / NT;         // 16-byte K chunks per thread
  static constexpr int VCH = (BC / 4) * (D / 4) / NT; // 4x4 V blocks per thread
  static constexpr int LDS_BYTES = 2 * (KBUF + VBUF) * 2;
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(KCH * NT * 8 == BC * D, "K tile must split evenly over the threads");
  static_assert(VCH * NT * 16 == BC * D, "V tile must split evenly over the threads");
};

template <typename TT, int D, int BC, int NW, int WPE, bool CAUSAL, bool VARLEN>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(WPE, WPE)))
attn_fwd_kernel(FwdParams p) {
  using C = TileCfg<D, BC, NW>;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  // ---- work item -> (head, query tile) -------------------------------------
  const int work = xcd_remap(blockIdx.x, p.n_work);
  const int head = work / p.tiles_per_head;
  const int t = work - head * p.tiles_per_head;
  int64_t q_row0, k_row0;
  int q_len, k_len, qt;
  if constexpr (!VARLEN) {
    q_len = p.Nq;
    k_len = p.Nk;
    q_row0 = (int64_t)head * p.Nq;
    k_row0 = (int64_t)head * p.Nk;
    qt = CAUSAL ? (p.tiles_per_head - 1 - t) : t;
  } else {
    int acc = 0, seq = -1, qb = 0, qe = 0, nts = 0;
    for (int s = 0; s < p.B; ++s) {
      const int a = min(max(p.cu_q[s], 0), p.Nq);
      const int b = min(max(p.cu_q[s + 1], a), p.Nq);
      const int nt = (b - a + C::BR - 1) / C::BR;
      if (t < acc + nt) {
        seq = s; qb = a; qe = b; nts = nt;
        break;
      }
      acc += nt;
    }
    if (seq < 0) return;  // surplus workgroup (the grid is an upper bound)
    const int lt = t - acc;
    qt = CAUSAL ? (nts - 1 - lt) : lt;
    const int kb = min(max(p.cu_k[seq], 0), p.Nk);
    const int ke = min(max(p.cu_k[seq + 1], kb), p.Nk);
    q_len = qe - qb;
    k_len = ke - kb;
    q_row0 = (int64_t)head * p.Nq + qb;
    k_row0 = (int64_t)head * p.Nk + kb;
  }
  const int q0 = qt * C::BR;

  const uint16_t* __restrict__ Qp = (const uint16_t*)p.q + q_row0 * D;
  const uint16_t* __restrict__ Kp = (const uint16_t*)p.k + k_row0 * D;
  const uint16_t* __restrict__ Vp = (const uint16_t*)p.v + k_row0 * D;

  const int tid = threadIdx.x;
  const int wv = tid >> 6, lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int qw0 = q0 + wv * 32;  // first query row of this wave
  const int my_q = qw0 + c;      // this lane's query row
  const bool q_ok = my_q < q_len;

  // ---- Q fragments: B operand of S^T = K Q^T, kept for the whole kernel ---
  uint4 qf[C::KS];
  {
    const uint16_t* qrow = Qp + (int64_t)(q_ok ? my_q : 0) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = q_ok ? *(const uint4*)(qrow + ks * 16) : zero4();
  }

  // ---- key tiles this workgroup / wave needs ------------------------------
  int n_kt = (k_len + BC - 1) / BC;
  if (CAUSAL) {
    const int last_q = min(q0 + C::BR, q_len) - 1;
    n_kt = min(n_kt, last_q / BC + 1);
  }
  int wave_kt = n_kt;
  if (qw0 >= q_len) {
    wave_kt = 0;
  } else if (CAUSAL) {
    const int wave_last_q = min(qw0 + 31, q_len - 1);
    wave_kt = min(n_kt, wave_last_q / BC + 1);
  }

  uint16_t* const ldsK = lds;
  uint16_t* const ldsV = lds + 2 * C::KBUF;

  uint4 kr[C::KCH];
  uint2 vr[C::VCH][4];

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const int ch = tid + i * C::NT;
      const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
      const int key = kt * BC + row;
      kr[i] = key < k_len ? *(const uint4*)(Kp + (int64_t)key * D + col) : zero4();
    }
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) {
      const int ch = tid + i * C::NT;
      const int kg = ch / (D / 4), dg = ch % (D / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kt * BC + 4 * kg + r;
        vr[i][r] = key < k_len ? *(const uint2*)(Vp + (int64_t)key * D + 4 * dg) : make_uint2(0u, 0u);
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* kb = ldsK + buf * C::KBUF;
    uint16_t* vb = ldsV + buf * C::VBUF;
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const int ch = tid + i * C::NT;
      const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
      *(uint4*)(kb + row * C::KP + col) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) {
      const int ch = tid + i * C::NT;
      const int kg = ch / (D / 4), dg = ch % (D / 4);
      uint16_t* dst = vb + (4 * dg) * C::VP + vt_pos(4 * kg);
      // 4 keys x 4 channels -> for each channel, the 4 keys as one 8-byte word
      *(uint2*)(dst + 0 * C::VP) = make_uint2(lo_halves(vr[i][0].x, vr[i][1].x), lo_halves(vr[i][2].x, vr[i][3].x));
      *(uint2*)(dst + 1 * C::VP) = make_uint2(hi_halves(vr[i][0].x, vr[i][1].x), hi_halves(vr[i][2].x, vr[i][3].x));
      *(uint2*)(dst + 2 * C::VP) = make_uint2(lo_halves(vr[i][0].y, vr[i][1].y), lo_halves(vr[i][2].y, vr[i][3].y));
      *(uint2*)(dst + 3 * C::VP) = make_uint2(hi_halves(vr[i][0].y, vr[i][1].y), hi_halves(vr[i][2].y, vr[i][3].y));
    }
  };

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  const float cs = p.c;
  float M = -INFINITY;  // integer reference max (base 2) of this lane's row
  float l = 0.f;        // this lane's partial row sum (its half of the keys)
  f32x16_t oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16_t{};

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) load_tile(kt + 1);

    if (kt < wave_kt) {
      const uint16_t* kb = ldsK + buf * C::KBUF;
      const uint16_t* vb = ldsV + buf * C::VBUF;

      // S^T = K Q^T for the tile
      f32x16_t s[C::MB];
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        s[mb] = f32x16_t{};
        const uint16_t* krow = kb + (mb * 32 + c) * C::KP + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) s[mb] = mfma32(TT{}, *(const uint4*)(krow + ks * 16), qf[ks], s[mb]);
      }

      const int key0 = kt * BC;
      const bool need_mask = (key0 + BC > k_len) || (CAUSAL && key0 + BC - 1 > qw0);
      float tmax = -INFINITY;
      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + mb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            const bool ok = key < k_len && (!CAUSAL || key <= my_q);
            s[mb][i] = ok ? s[mb][i] * cs : -INFINITY;
            tmax = fmaxf(tmax, s[mb][i]);
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[mb][i]);
        tmax *= cs;
      }
      tmax = max_halves(tmax);
      const float m_new = fmaxf(M, __builtin_ceilf(tmax));
      if (__any(m_new > M)) {
        const float alpha = (m_new == M) ? 1.f : __builtin_amdgcn_exp2f(M - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
      M = m_new;
      const float m_use = (M == -INFINITY) ? 0.f : M;

      float rs = 0.f;
      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s[mb][i] = __builtin_amdgcn_exp2f(s[mb][i] - m_use);
            rs += s[mb][i];
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s[mb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][i], cs, -m_use));
            rs += s[mb][i];
          }
      }
      l += rs;

      // P^T as the B operand of O^T += V^T P^T (keys of register i of block mb:
      // 8*(i/4) + 4*hh + i%4, which is the order vt_pos lays V^T out in).
      //
      // Rows whose weight so far sits on few keys (small l) have large |O|,
      // where the 16-bit rounding of P would show.  For them the residual
      // p - round16(p) goes through a second product, so the weights carry
      // about 16 more bits; diffuse rows average the rounding out and skip it.
      uint4 pf[C::MB][2];
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int b = 8 * h2;
          pf[mb][h2] = make_uint4(pack2(TT{}, s[mb][b + 0], s[mb][b + 1]), pack2(TT{}, s[mb][b + 2], s[mb][b + 3]),
                                  pack2(TT{}, s[mb][b + 4], s[mb][b + 5]), pack2(TT{}, s[mb][b + 6], s[mb][b + 7]));
        }
      if (__any(l < kSplitBelow)) {
        uint4 pl[C::MB][2];
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int b = 8 * h2;
            pl[mb][h2] = make_uint4(residual2(TT{}, pf[mb][h2].x, s[mb][b + 0], s[mb][b + 1]),
                                    residual2(TT{}, pf[mb][h2].y, s[mb][b + 2], s[mb][b + 3]),
                                    residual2(TT{}, pf[mb][h2].z, s[mb][b + 4], s[mb][b + 5]),
                                    residual2(TT{}, pf[mb][h2].w, s[mb][b + 6], s[mb][b + 7]));
          }
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const uint16_t* vrow = vb + (db * 32 + c) * C::VP + 8 * hh;
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const uint4 va = *(const uint4*)(vrow + mb * 32 + 16 * h2);
              oacc[db] = mfma32(TT{}, va, pf[mb][h2], oacc[db]);
              oacc[db] = mfma32(TT{}, va, pl[mb][h2], oacc[db]);
            }
        }
      } else {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const uint16_t* vrow = vb + (db * 32 + c) * C::VP + 8 * hh;
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
              oacc[db] = mfma32(TT{}, *(const uint4*)(vrow + mb * 32 + 16 * h2), pf[mb][h2], oacc[db]);
        }
      }
    }

    if (kt + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O / l, lse = (M + log2 l) ln 2 -----------------------
  const float l_tot = sum_halves(l);
  if (q_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = (uint16_t*)p.o + (q_row0 + my_q) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dcol = db * 32 + 8 * g + 4 * hh;
        *(uint2*)(orow + dcol) = make_uint2(pack2(TT{}, oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                                            pack2(TT{}, oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv));
      }
    if (hh == 0) p.lse[q_row0 + my_q] = l_tot > 0.f ? (M + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename TT, int D, int BC, int NW, int WPE, bool CAUSAL, bool VARLEN>
hipError_t launch_one(const FwdParams& p, hipStream_t st) {
  using C = TileCfg<D, BC, NW>;
  auto kern = attn_fwd_kernel<TT, D, BC, NW, WPE, CAUSAL, VARLEN>;
  static bool attr_set = false;  // idempotent; a benign race between threads
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(p.n_work), dim3(C::NT), C::LDS_BYTES, st, p);
  return hipGetLastError();
}

// Tile configuration per head dimension: key rows per tile BC, waves per
// workgroup NW (query rows BR = 32 NW), waves per SIMD the registers allow.
template <int D> struct FwdTile;
template <> struct FwdTile<64> { static constexpr int BC = 64, NW = 4, WPE = 2; };
template <> struct FwdTile<128> { static constexpr int BC = 64, NW = 8, WPE = 2; };
template <> struct FwdTile<256> { static constexpr int BC = 32, NW = 4, WPE = 1; };

template <typename TT, bool CAUSAL, bool VARLEN>
hipError_t launch_d(int d, const FwdParams& p, hipStream_t st) {
  switch (d) {
    case 64: return launch_one<TT, 64, FwdTile<64>::BC, FwdTile<64>::NW, FwdTile<64>::WPE, CAUSAL, VARLEN>(p, st);
    case 128: return launch_one<TT, 128, FwdTile<128>::BC, FwdTile<128>::NW, FwdTile<128>::WPE, CAUSAL, VARLEN>(p, st);
    case 256: return launch_one<TT, 256, FwdTile<256>::BC, FwdTile<256>::NW, FwdTile<256>::WPE, CAUSAL, VARLEN>(p, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename TT>
hipError_t launch_t(int d, bool causal, bool varlen, const FwdParams& p, hipStream_t st) {
  if (causal) return varlen ? launch_d<TT, true, true>(d, p, st) : launch_d<TT, true, false>(d, p, st);
  return varlen ? launch_d<TT, false, true>(d, p, st) : launch_d<TT, false, false>(d, p, st);
}

}  // namespace

int fwd_block_rows(int dtype, int d) {
  if (dtype == 2) return fwd_fp8_block_rows();
  switch (d) {
    case 64: return 32 * FwdTile<64>::NW;
    case 128: return 32 * FwdTile<128>::NW;
    default: return 32 * FwdTile<256>::NW;
  }
}

hipError_t launch_fwd(int dtype, int d, bool causal, bool varlen, const FwdParams& p, hipStream_t st) {
  if (dtype == 0) return launch_t<f16_t>(d, causal, varlen, p, st);
  return launch_t<bf16_t>(d, causal, varlen, p, st);
}

}  // namespace attn
