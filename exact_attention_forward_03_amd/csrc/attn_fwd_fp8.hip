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
// query rows, K/V tiles streamed from global memory straight into a ring of
// LDS slots, S^T = K Q^T so P stays in registers), with these differences:
//   * 32x32x64 e4m3 MFMA, fp32 accumulation; head dimension d = 64, 128 or
//     256; key tiles of 128 rows (64 at d = 256, to fit two waves per SIMD),
//     so each tile lies within one 128-row tile of K and V scales;
//   * scores t = acc * (scale log2 e * s_q * s_k) in base 2; M = ceil(max t)
//     per row (an integer, so rescaling O and l is exact), updated once per
//     key tile;
//   * P is rounded to e4m3 as e4m3(2^(t - M + 8) * w), w = s_v(tile) /
//     max_tiles s_v: the V tile's scale is folded into the exponent, so the
//     PV product needs no per-tile correction of O and the codes stay <= 256;
//     l sums the unrounded 2^(t - M) and O = (max s_v) 2^-8 sum P8 v8 / l;
//   * V stays row-major in LDS; the V^T operand comes from the 8-bit
//     transposing LDS read (ds_read_b64_tr_b8: within a 16-lane group, lane
//     i receives byte i % 8 of the 8-byte pieces read by lanes 2j + i / 8),
//     so each lane reads the 8 keys of one V column that its P bytes need;
//   * variable-length batches restart the scale tiles at every sequence
//     (the work item is (head, sequence, query tile));
//   * dense causal launches run pairs of query tiles of equal total work
//     per workgroup, as the fp16/bf16 kernel does.
#include "attn_device.h"
#include "attn_params.h"
#include "attn_sched.h"

namespace attn {
namespace {

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kScaleRows = 128;  // rows per Q/K/V scale
constexpr int kFp8Pre = 4;    // K fragments (two reads each) in flight ahead of their MFMA
constexpr int kFp8PvPre = 3;  // V^T fragments (four reads each): at most 12 LDS reads in flight,
                              // within what the 4-bit lgkmcnt counter can track

// Tile geometry per head dimension: key rows per tile, waves per workgroup,
// ring slots.  4-wave workgroups with a 2-slot ring, two per CU (see the
// launch).  d = 256 takes 64-key tiles: with 128 keys the scores (64
// registers) next to O's 128 accumulators and Q's 32 do not fit the 256
// registers of two waves per SIMD.
// KPRE / VPRE: K and V^T fragments in flight ahead of their MFMAs (fewer at
// d = 256, where the registers are short).
template <int D> struct Fp8Tile;
template <> struct Fp8Tile<64> { static constexpr int BC = 128, NW = 4, NS = 2, KPRE = kFp8Pre, VPRE = kFp8PvPre; };
template <> struct Fp8Tile<128> { static constexpr int BC = 128, NW = 4, NS = 2, KPRE = kFp8Pre, VPRE = kFp8PvPre; };
template <> struct Fp8Tile<256> { static constexpr int BC = 64, NW = 4, NS = 2, KPRE = 1, VPRE = 1; };

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void fp8_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Physical 16-byte chunk (of D/16 per row) of logical chunk ch in row r.
// The LDS serves 256 bytes (64 banks) per cycle.  K fragment reads: 16
// lanes read 16 consecutive rows at one logical chunk; 256/D rows share a
// bank line, so the chunk is XOR-ed with the row's bank-line index (mod the
// chunk count): the 16 reads hit 16 different 16-byte bank slots.  V
// transposing reads: 32 lanes read 8 rows {0..3, 8..11} + 4h (plus a
// multiple of 16) at two neighbouring chunks, 8 bytes each; the XOR below
// spreads those 32 pieces over all 64 banks (d = 128: 2 bit1 + 4 bit3 of the
// row; d = 64: 2 bit3; d = 256: 2 (r mod 4) + 8 bit3).  Both depend on the
// row mod 16 only.
template <int D>
__device__ __forceinline__ int k8_chunk(int r, int ch) {
  constexpr int CH = D / 16, RPL = D >= 256 ? 1 : 256 / D;
  return ch ^ ((r / RPL) % CH);
}
template <int D>
__device__ __forceinline__ int v8_chunk(int r, int ch) {
  if constexpr (D == 64) return ch ^ (((r >> 3) & 1) << 1);
  else if constexpr (D == 128) return ch ^ (((r >> 1) & 1) << 1) ^ (((r >> 3) & 1) << 2);
  else return ch ^ ((r & 3) << 1) ^ (((r >> 3) & 1) << 3);
}

// The first conversion's "old" operand (whose upper half it keeps) is a's
// own bits: the second conversion overwrites that half, and a dies here, so
// the result takes a's register and needs no zeroing move.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
// The same with the register of `old` (a value that dies here) as the home of
// the result.
__device__ __forceinline__ uint32_t pack4_e4m3_into(float a, float b, float c, float d, float old) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, old), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// D head dimension, BC key rows per tile, NW waves per workgroup (32 query
// rows each), NS LDS ring slots.  VARLEN: a packed batch [H, T, d] with
// cu_seqlens; the work item is (head, sequence, query tile) and the scales of
// sequence s start at entry floor(cu[s] / 128) + s of the head's
// ceil(T / 128) + B entries (sched::slot_tile).
template <int D, int BC, bool CAUSAL, int NW, int NS, bool VARLEN, bool SPLIT>
__device__ __forceinline__ void fp8_body(const FwdParams& p, const int work) {
  constexpr int SC = kScaleRows;
  constexpr int kRowB = D;               // bytes per K/V row
  constexpr int kTileB = BC * kRowB;     // bytes per K or V tile
  constexpr int kLoads = kTileB / 1024;  // 1 KiB direct-to-LDS loads per tile
  constexpr int CH = D / 16;             // 16-byte chunks per row
  constexpr int RPB = 1024 / D;          // rows per 1 KiB block
  constexpr int BR = NW * 32;
  static_assert(SC % BR == 0 && SC % BC == 0, "query and key tiles lie within one scale tile");
  constexpr int KS = D / 64;    // MFMA k-steps of S^T
  constexpr int MB = BC / 32;   // 32-key blocks per tile
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  constexpr int PG = BC / 64;   // MFMA k-steps of O^T (64 keys each)
  constexpr int LPW = kLoads / NW;  // loads per wave per K (or V) tile
  constexpr int LPT = 2 * LPW;      // per tile, K and V
  static_assert(kLoads % NW == 0, "each wave issues the same number of tile loads");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds8[];

  static_assert(!(SPLIT && VARLEN), "key chunks are for dense batches");
  int head, qt, q_len, k_len;
  int k_off = 0, split = 0;  // key chunks: first key of the chunk, chunk index
  int64_t q_row0, k_row0, sq0, sk0;  // first rows of the (sequence,) head; its first scale entries
  if constexpr (!VARLEN) {
    // work = (head * n_split + chunk) * tiles_per_head + t (n_split = 1 without chunks)
    const int hs = work / p.tiles_per_head;
    const int t = work - hs * p.tiles_per_head;
    head = SPLIT ? hs / p.n_split : hs;
    qt = CAUSAL ? (p.tiles_per_head - 1 - t) : t;
    q_len = p.Nq;
    k_len = p.Nk;
    if constexpr (SPLIT) {
      // chunks of whole scale tiles (split_len is a multiple of SC)
      split = hs - head * p.n_split;
      k_off = (int)min((int64_t)split * p.split_len, (int64_t)p.Nk);
      k_len = (int)min((int64_t)p.split_len, (int64_t)p.Nk - k_off);
    }
    q_row0 = (int64_t)head * p.Nq;
    k_row0 = (int64_t)head * p.Nk + k_off;
    sq0 = (int64_t)head * ((q_len + SC - 1) / SC);
    sk0 = (int64_t)head * ((p.Nk + SC - 1) / SC) + k_off / SC;
  } else {
    // t: a slot of the head's 128-row query tiles (sched::slot_tile); the
    // scale entries of a packed batch use the same slots, so the sequence's
    // first q and k scale entries follow from its first rows
    head = work / p.tiles_per_head;
    const int t = work - head * p.tiles_per_head;
    static_assert(BR == SC, "query tiles are the scale tiles");
    sched::SlotTile st;
    if (!sched::find_tile<BR>(p.cu_q, p.B, p.Nq, p.cu_k, p.Nk, t, st)) return;  // surplus slot (the grid is an upper bound)
    const int nts = (st.e - st.a + BR - 1) / BR;
    qt = CAUSAL ? (nts - 1 - st.j) : st.j;
    q_len = st.e - st.a;
    k_len = st.oe - st.oa;
    q_row0 = (int64_t)head * p.Nq + st.a;
    k_row0 = (int64_t)head * p.Nk + st.oa;
    sq0 = (int64_t)head * ((p.Nq + SC - 1) / SC + p.B) + sched::first_slot<SC>(st.a, st.seq);
    sk0 = (int64_t)head * ((p.Nk + SC - 1) / SC + p.B) + sched::first_slot<SC>(st.oa, st.seq);
  }
  const int q0 = qt * BR;
  const int nks = (k_len + SC - 1) / SC;
  const float* __restrict__ sk = p.k_scale + sk0;
  const float* __restrict__ sv = p.v_scale + sk0;

  const uint8_t* __restrict__ Qp = (const uint8_t*)p.q + q_row0 * D;
  const uint8_t* __restrict__ Kp = (const uint8_t*)p.k + k_row0 * D;
  const uint8_t* __restrict__ Vp = (const uint8_t*)p.v + k_row0 * D;

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  // the lane index through an empty asm: a launch that runs two bodies one
  // after the other then forms the per-lane offsets in each body, rather
  // than once for both, live (and spilled) across the first
  int lane = tid & 63;
  asm volatile("" : "+v"(lane));
  const int c = lane & 31, hh = lane >> 5;
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
  const float sq = wave_live ? p.q_scale[sq0 + qw0 / SC] : 0.f;

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
  if (CAUSAL) {
    // last key (within the chunk) that some row of the workgroup sees
    const int last = min(q0 + BR, q_len) - 1 - k_off;
    n_kt = last < 0 ? 0 : min(n_kt, last / BC + 1);
  }
  int wave_kt = n_kt;
  if (!wave_live) {
    wave_kt = 0;
  } else if (CAUSAL) {
    const int last = min(qw0 + 31, q_len - 1) - k_off;
    wave_kt = last < 0 ? 0 : min(n_kt, last / BC + 1);
  }

  uint8_t* const ldsK = lds8;
  uint8_t* const ldsV = lds8 + NS * kTileB;

  float M = -INFINITY, l = 0.f;
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};

  // Direct-to-LDS load of one tile into ring slot `buf`: the wave's i-th
  // instruction fills 1 KiB block i * NW + wv (RPB rows) of K and of V; lane
  // l writes physical chunk l % CH of row RPB * block + l / CH and fetches
  // the logical chunk stored there.  The rows come through buffer resources
  // based at the tile's first key: the swizzles read the row mod 16, which
  // does not depend on i, so a lane's byte offset is the same for every
  // load and tile and the block offset is a scalar.  The resources cover only
  // the tile's keys; a last tile that runs past them re-reads the last key
  // (finite codes, masked) through per-lane clamped offsets.
  static_assert((NW * RPB) % 16 == 0, "block rounds span whole swizzle periods");
  auto load_tile = [&](int kt, uint8_t* kdst, uint8_t* vdst) {
    const int rows = min(BC, k_len - kt * BC);  // >= 1: only tiles holding keys are loaded
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kp + (int64_t)kt * BC * kRowB), 0, rows * kRowB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Vp + (int64_t)kt * BC * kRowB), 0, rows * kRowB, kBufferFlags);
    const int r0 = wv * RPB + lane / CH;  // row of the lane's first block; later blocks agree mod 16
    if (rows == BC) {
      const uint32_t offk = (uint32_t)((lane / CH) * kRowB + k8_chunk<D>(r0, lane % CH) * 16);
      const uint32_t offv = (uint32_t)((lane / CH) * kRowB + v8_chunk<D>(r0, lane % CH) * 16);
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int blk = i * NW + wv;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kdst + blk * 1024), 16, offk,
                                                 (uint32_t)(blk * 1024), 0, 0);
      }
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int blk = i * NW + wv;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vdst + blk * 1024), 16, offv,
                                                 (uint32_t)(blk * 1024), 0, 0);
      }
    } else {
      // the lane index through an empty asm: the per-lane rows and chunks of
      // this rare path are then computed here, not hoisted out of the tile
      // loop to occupy registers (or scratch) for the whole kernel
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int blk = i * NW + wv;
        const int r = blk * RPB + ln / CH;
        const uint32_t off = (uint32_t)(min(r, rows - 1) * kRowB + k8_chunk<D>(r, ln % CH) * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kdst + blk * 1024), 16, off, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int blk = i * NW + wv;
        const int r = blk * RPB + ln / CH;
        const uint32_t off = (uint32_t)(min(r, rows - 1) * kRowB + v8_chunk<D>(r, ln % CH) * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vdst + blk * 1024), 16, off, 0, 0, 0);
      }
    }
  };

  // S^T of the tile in slot kbuf: step i = (32-key block i % MB, k-step i / MB)
  auto compute_s = [&](const uint8_t* kb, f32x16_t (&s)[MB]) {
    constexpr int N = MB * KS;
    auto frag = [&](int i, uint4 (&f)[2]) {
      const int r = (i % MB) * 32 + c;
      const int ch = 4 * (i / MB) + 2 * hh;
      f[0] = *(const uint4*)(kb + r * kRowB + k8_chunk<D>(r, ch) * 16);
      f[1] = *(const uint4*)(kb + r * kRowB + k8_chunk<D>(r, ch + 1) * 16);
    };
    constexpr int PRE = Fp8Tile<D>::KPRE < N ? Fp8Tile<D>::KPRE : N;
    uint4 fr[PRE][2];
#pragma unroll
    for (int i = 0; i < PRE; ++i) frag(i, fr[i]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) s[mb] = f32x16_t{};
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint4 a0 = fr[i % PRE][0], a1 = fr[i % PRE][1];
      s[i % MB] = mfma32_fp8(a0, a1, qf[i / MB][0], qf[i / MB][1], s[i % MB]);
      if (i + PRE < N) frag(i + PRE, fr[i % PRE]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // O^T += V^T P^T for the tile in slot vbuf.  Step i = (output block
  // i % DB, 64-key step i / DB).  MFMA k-index 32 h + j of lane half h holds
  // key 64 g + 32 (j / 16) + 8 ((j % 16) / 4) + 4 h + j % 4 (the order of P's
  // registers); the four transposing reads m = 0..3 of a fragment deliver
  // k-indices 8m .. 8m+7.  In 16-lane group G (h = G / 2), source lane s
  // reads row key(8m + s / 2) at columns 32 db + 16 (G % 2) + 8 (s % 2) ..+8.
  // The swizzle of row r reads bits 1 and 3 of r only, which come from the
  // lane's part of the row (the rest is a multiple of 16): each lane's byte
  // offset within a tile is one of DB loop-invariant values (one per output
  // block), and the row steps are immediate offsets of the reads.
  // At d = 256 the eight offsets would not fit beside O's 128 accumulators:
  // there the lane keeps its row-and-half base and the XOR key of its row
  // (v8_chunk flips chunk bits 1..3 only, so chunk 2 db + g of row lr sits
  // at 2 (db ^ key) + g) and forms each offset when the fragment is read.
  constexpr bool kVlaneArray = D < 256;
  uint32_t vlane[kVlaneArray ? DB : 1];
  uint32_t vbase = 0, vkey = 0;
  {
    const int G = lane >> 4, s16 = lane & 15, b = s16 >> 1;
    const int lr = 8 * (b >> 2) + 4 * hh + (b & 3);  // the lane's row within 16
    if constexpr (kVlaneArray) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        vlane[db] = (uint32_t)(lr * kRowB + v8_chunk<D>(lr, 2 * db + (G & 1)) * 16 + 8 * (s16 & 1));
    } else {
      vbase = (uint32_t)(lr * kRowB + (G & 1) * 16 + 8 * (s16 & 1));
      vkey = (uint32_t)(v8_chunk<D>(lr, 0) >> 1);
    }
  }
  auto pv_pass = [&](const uint8_t* vb, const uint4 (&pp)[PG][2]) {
    // the key through an empty asm, so that the offsets are formed here and
    // not hoisted out of the tile loop (eight registers again)
    uint32_t vk = vkey;
    if constexpr (!kVlaneArray) asm volatile("" : "+v"(vk));
    auto v_offset = [&](int db) -> uint32_t {
      if constexpr (kVlaneArray) return vlane[db];
      else return vbase + 32u * ((uint32_t)db ^ vk);
    };
    constexpr int N = DB * PG;
    auto frag = [&](int i, uint4 (&f)[2]) {
      const int db = i % DB, g = i / DB;
      const uint8_t* base = vb + v_offset(db);
      uint32_t w[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int rstep = 64 * g + 32 * (m >> 1) + 16 * (m & 1);  // multiple of 16 rows
        const i32x2_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(base + rstep * kRowB));
        w[2 * m] = (uint32_t)x[0];
        w[2 * m + 1] = (uint32_t)x[1];
      }
      f[0] = make_uint4(w[0], w[1], w[2], w[3]);
      f[1] = make_uint4(w[4], w[5], w[6], w[7]);
    };
    constexpr int PRE = Fp8Tile<D>::VPRE < N ? Fp8Tile<D>::VPRE : N;
    uint4 fr[PRE][2];
#pragma unroll
    for (int i = 0; i < PRE; ++i) frag(i, fr[i]);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int db = i % DB, g = i / DB;
      const uint4 a0 = fr[i % PRE][0], a1 = fr[i % PRE][1];
      oacc[db] = mfma32_fp8(a0, a1, pp[g][0], pp[g][1], oacc[db]);
      if (i + PRE < N) frag(i + PRE, fr[i % PRE]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // prologue: tiles 0 .. NS-2 in flight (tile j in ring slot j % NS)
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_kt) load_tile(j, ldsK + j * kTileB, ldsV + j * kTileB);

  int slot = 0;  // ring slot of tile kt
  for (int kt = 0; kt < n_kt; ++kt) {
    if (kt + NS - 2 < n_kt) fp8_wait_vm<(NS - 2) * LPT>();
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // refill the slot tile kt-1 used (every wave is past it now); a live
    // wave issues these loads after its S chain, which then starts at once
    // after the barrier (+4-6 % measured over loads first).  The slot filled
    // and the slot read are different, passed as restrict pointers: the
    // compiler then knows the reads do not depend on the direct-to-LDS loads
    // just issued and does not wait for them (it would otherwise wait for
    // every outstanding load before the next LDS read).  The explicit vmcnt
    // wait and barrier above order the reads after the loads of earlier
    // steps.
    const bool refill = kt + NS - 1 < n_kt;
    const int fs = slot == 0 ? NS - 1 : slot - 1;
    with_disjoint(ldsK + fs * kTileB, ldsV + fs * kTileB, ldsK + slot * kTileB, ldsV + slot * kTileB,
                  [&](uint8_t* kw, uint8_t* vw, const uint8_t* kr, const uint8_t* vr) __attribute__((always_inline)) {
      if (kt >= wave_kt && refill) load_tile(kt + NS - 1, kw, vw);

      if (kt < wave_kt) {
        // the tile's scales through the scalar cache: a vector load here
        // would make the compiler wait for the tile loads issued before it
        const int kst = kt * BC / SC;  // the tile's scale entry
        const float cs = p.c * sq * load_uniform(sk, kst);
        const float svt = load_uniform(sv, kst);
        // log2 of 2^8 w: P codes are e4m3(2^(t - M) * 2^8 * s_v / max s_v).
        // With 2^8 w <= 2^-11 every code of the tile is 0 (values <= 2^-10
        // round to 0): the tile then skips the PV product, and its
        // exponentials are taken with bias 8 so that l still gets its mass.
        // That covers a V scale of 0 (bias -inf).
        const float bias_w = 8.f + (svt > 0.f ? __log2f(svt) - lsv_max : -INFINITY);
        const bool pv_zero = !(bias_w >= -11.f);
        const float bias = pv_zero ? 8.f : bias_w;

        f32x16_t s[MB];
        compute_s(kr, s);
        if (refill) load_tile(kt + NS - 1, kw, vw);

        const int key0 = kt * BC;
        const bool need_mask = (key0 + BC > k_len) || (CAUSAL && k_off + key0 + BC - 1 > qw0);
        float t4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (need_mask) {
  #pragma unroll
          for (int mb = 0; mb < MB; ++mb)
  #pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = key0 + mb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
              const bool ok = key < k_len && (!CAUSAL || k_off + key <= my_q);
              s[mb][i] = ok ? s[mb][i] * cs : -INFINITY;
              t4[i & 3] = fmaxf(t4[i & 3], s[mb][i]);
            }
        } else {
  #pragma unroll
          for (int mb = 0; mb < MB; ++mb)
  #pragma unroll
            for (int i = 0; i < 16; ++i) t4[i & 3] = fmaxf(t4[i & 3], s[mb][i]);
        }
        float tmax = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
        if (!need_mask) tmax *= cs;  // scales are >= 0
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

        float r4[4] = {0.f, 0.f, 0.f, 0.f};
        if (need_mask) {
  #pragma unroll
          for (int mb = 0; mb < MB; ++mb)
  #pragma unroll
            for (int i = 0; i < 16; ++i) {
              s[mb][i] = __builtin_amdgcn_exp2f(s[mb][i] + off);
              r4[i & 3] += s[mb][i];
            }
        } else {
  #pragma unroll
          for (int mb = 0; mb < MB; ++mb)
  #pragma unroll
            for (int i = 0; i < 16; ++i) {
              s[mb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][i], cs, off));
              r4[i & 3] += s[mb][i];
            }
        }
        const float rs = (r4[0] + r4[1]) + (r4[2] + r4[3]);
        // rs sums 2^(t - M) * 2^bias; l keeps the unweighted sum
        l += rs * __builtin_amdgcn_exp2f(-bias);
        if (pv_zero) return;  // wave-uniform: the tile's V scale is the same for every lane

        // P codes: step g takes key blocks 2g (bytes 0..15) and 2g+1 (16..31)
        uint4 pp[PG][2];
  #pragma unroll
        for (int g = 0; g < PG; ++g) {
          const f32x16_t& a = s[2 * g];
          const f32x16_t& bb = s[2 * g + 1];
          // word k of the operand goes to the register of a[k], the first
          // eight of the block's 16 consecutive registers, each dead by then:
          // the MFMA operand is then built in place, with no copies
          pp[g][0] = make_uint4(pack4_e4m3_into(a[0], a[1], a[2], a[3], a[0]),
                                pack4_e4m3_into(a[4], a[5], a[6], a[7], a[1]),
                                pack4_e4m3_into(a[8], a[9], a[10], a[11], a[2]),
                                pack4_e4m3_into(a[12], a[13], a[14], a[15], a[3]));
          pp[g][1] = make_uint4(pack4_e4m3_into(bb[0], bb[1], bb[2], bb[3], a[4]),
                                pack4_e4m3_into(bb[4], bb[5], bb[6], bb[7], a[5]),
                                pack4_e4m3_into(bb[8], bb[9], bb[10], bb[11], a[6]),
                                pack4_e4m3_into(bb[12], bb[13], bb[14], bb[15], a[7]));
        }
        pv_pass(vr, pp);
      }
    });
    slot = (slot + 1 == NS) ? 0 : slot + 1;
  }

  const float l_tot = sum_halves(l);
  if (SPLIT && q_ok) {
    // the chunk's normalised O and its lse, fp32, for the merge kernel
    const float f = l_tot > 0.f ? sv_max * (1.f / 256.f) / l_tot : 0.f;
    const int64_t prow = (int64_t)split * p.B * p.H * p.Nq + q_row0 + my_q;
    float* orow = p.o_part + prow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(orow + db * 32 + 8 * g + 4 * hh) =
            make_float4(oacc[db][4 * g + 0] * f, oacc[db][4 * g + 1] * f, oacc[db][4 * g + 2] * f,
                        oacc[db][4 * g + 3] * f);
    if (hh == 0) p.lse_part[prow] = l_tot > 0.f ? (M + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else if (q_ok) {
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

// The kernel: one work item, or for dense causal launches a pair of query
// tiles of equal total work, one after the other: tile t of head h and tile
// T-1-t of head h + heads/2 (an even head count), else tiles t and T-1-t of
// one head; p.n_work counts pairs then.
template <int D, int BC, bool CAUSAL, int NW, int NS, bool VARLEN, bool SPLIT>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(2, 2)))
attn_fwd_fp8_kernel(FwdParams p) {
  const int w = xcd_remap(blockIdx.x, p.n_work);
  if constexpr (CAUSAL && !VARLEN && !SPLIT) {
    const int T = p.tiles_per_head, heads = p.B * p.H;
    if (heads % 2 == 0) {
      const int h = w / T, t = w - h * T;
      fp8_body<D, BC, CAUSAL, NW, NS, VARLEN, SPLIT>(p, h * T + t);
      __syncthreads();
      fp8_body<D, BC, CAUSAL, NW, NS, VARLEN, SPLIT>(p, (h + heads / 2) * T + (T - 1 - t));
    } else {
      const int half = (T + 1) / 2;
      const int head = w / half, t = w - head * half;
      fp8_body<D, BC, CAUSAL, NW, NS, VARLEN, SPLIT>(p, head * T + t);
      if (T - 1 - t != t) {
        __syncthreads();
        fp8_body<D, BC, CAUSAL, NW, NS, VARLEN, SPLIT>(p, head * T + (T - 1 - t));
      }
    }
  } else {
    fp8_body<D, BC, CAUSAL, NW, NS, VARLEN, SPLIT>(p, w);
  }
}

template <int D, bool CAUSAL, bool VARLEN, bool SPLIT = false>
hipError_t launch_fp8(const FwdParams& p, hipStream_t st) {
  constexpr int BC = Fp8Tile<D>::BC, NW = Fp8Tile<D>::NW, NS = Fp8Tile<D>::NS;
  constexpr int lds = 2 * NS * BC * D;
  auto kern = attn_fwd_fp8_kernel<D, BC, CAUSAL, NW, NS, VARLEN, SPLIT>;
  static bool attr_set = false;  // idempotent; a benign race between threads
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  FwdParams pp = p;
  if constexpr (CAUSAL && !VARLEN && !SPLIT) {
    const int64_t heads = p.n_work / p.tiles_per_head;
    pp.n_work = (int)(heads % 2 == 0 ? heads / 2 * p.tiles_per_head : heads * ((p.tiles_per_head + 1) / 2));
  }
  hipLaunchKernelGGL(kern, dim3(pp.n_work), dim3(NW * 64), lds, st, pp);
  return hipGetLastError();
}

// Configuration: 4-wave workgroups with a 2-slot ring (64 KiB), two per CU.
// The two waves that share a SIMD then belong to different workgroups, whose
// barriers are independent, so one wave's MFMA chains run while the other
// does its softmax work.  (One 8-wave workgroup per CU with a 4-slot ring
// puts two waves of the same workgroup on each SIMD, where the per-tile
// barrier keeps them in step: 631 -> 593 us at B2 H16 N8192 non-causal.)
// Causal launches also keep one workgroup's short diagonal tiles from
// idling the CU.

}  // namespace

int fwd_fp8_block_rows(bool causal) { return 32 * Fp8Tile<128>::NW; }

template <int D>
hipError_t launch_fp8_d(bool causal, bool varlen, bool split, const FwdParams& p, hipStream_t st) {
  static_assert(32 * Fp8Tile<D>::NW == 32 * Fp8Tile<128>::NW, "one query-tile height for every d");
  if (split) return causal ? launch_fp8<D, true, false, true>(p, st) : launch_fp8<D, false, false, true>(p, st);
  if (varlen) return causal ? launch_fp8<D, true, true>(p, st) : launch_fp8<D, false, true>(p, st);
  return causal ? launch_fp8<D, true, false>(p, st) : launch_fp8<D, false, false>(p, st);
}

hipError_t launch_fwd_fp8(int d, bool causal, bool varlen, bool split, const FwdParams& p, hipStream_t st) {
  switch (d) {
    case 64: return launch_fp8_d<64>(causal, varlen, split, p, st);
    case 128: return launch_fp8_d<128>(causal, varlen, split, p, st);
    case 256: return launch_fp8_d<256>(causal, varlen, split, p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
