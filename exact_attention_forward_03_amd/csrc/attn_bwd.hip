// Backward pass of exact attention for fp16/bf16 on gfx950 (CDNA4).
//
// The pages measure a backward pass ("FlashAttention-3" wiki page, the
// "Measured (H100 80GB SXM5)" table) without printing it; what it computes
// is the derivative of the forward definition ("Flash Attention 3：让 GPU
// 跑满的注意力计算", §1.2 and §2.2).  With P = softmax(scale Q K^T [+causal])
// and dO the gradient of the output:
//
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - delta),   delta_i = dO_i . O_i,
//   dQ = scale dS K,   dK = scale dS^T Q.
//
// Like the forward it never forms an N x N matrix in HBM: P is recomputed
// tile by tile from Q, K and the forward's lse (P = 2^(S scale log2 e -
// lse log2 e)), the same tiling as the forward (§2.1).  Three kernels:
//
// * delta: delta_i = sum_c dO_ic O_ic in fp32 (memory-bound; one read of O
//   and dO), written to a caller-provided fp32 buffer.
// * dK/dV: a workgroup owns 32*NW keys of one head, each wave 32 keys whose
//   K rows stay in registers as MFMA B operands (the workgroup's V rows are
//   loaded once into LDS).  Blocks of 32 query rows (Q, dO, lse, delta)
//   stream through an LDS ring (direct-to-LDS loads).  Per block and wave:
//   S = Q K^T and dP = dO V^T (operands read from LDS but K), the 32x32 P
//   and dS in registers, then dV^T += dO^T P^T and
//   dK^T += Q^T dS^T, whose A operands dO^T and Q^T come from the row-major
//   tiles by the transposing LDS read (ds_read_b64_tr_b16) and whose B
//   operands are P and dS exactly as the S accumulator holds them.
// * dQ: a workgroup owns 32*NW query rows, each wave 32 rows with Q and dO
//   in registers; K and V tiles stream through the ring as in the forward.
//   Per tile: S^T = K Q^T and dP^T = V dO^T, dS^T in registers, then
//   dQ^T += K^T dS^T (K^T by the transposing read).
//
// dQ is computed by its own pass over the keys rather than accumulated
// across dK/dV workgroups with atomics: the result is deterministic and no
// fp32 scratch is needed, at the cost of recomputing S and dP once more.
// Causal masking is top-left (key j visible to query i iff j <= i); blocks
// entirely outside the mask are skipped, diagonal blocks are masked per
// element.
#include "attn_device.h"
#include "attn_params.h"
#include "attn_sched.h"

namespace attn {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

template <int N>
__device__ __forceinline__ void bwd_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Row-major tiles of D 16-bit values per row, rows unpadded, the 16-byte
// chunks of row r XOR-permuted by r mod (chunks per row, at most 16).
template <int D>
struct Tile {
  static constexpr int ROWB = D * 2;
  static constexpr int CH = ROWB / 16;
  static constexpr int RPK = 1024 / ROWB;  // rows per 1 KiB direct-to-LDS load
  __device__ static int pos(int r, int ch) { return ch ^ (r & (CH >= 16 ? 15 : CH - 1)); }
  // MFMA operand with rows along the tile rows: lane l gets row `row`, the
  // 8 values of k-step ks of its half.
  __device__ static uint4 rows_frag(const uint8_t* t, int row, int ks, int hh) {
    return *(const uint4*)(t + row * ROWB + pos(row, 2 * ks + hh) * 16);
  }
  // MFMA operand with rows along the tile columns (the transpose of 32
  // columns x 16 rows): two transposing reads give lane l column
  // 32 db + l % 32 at rows 16 k16 + 8 (t / 4) + 4 (l / 32) + t % 4, t = 0..7,
  // the order in which a 32x32 accumulator holds its rows.
  __device__ static uint4 cols_frag(const uint8_t* t, int db, int k16, int lane) {
    const int hh = lane >> 5, g = (lane >> 4) & 1, s4 = lane & 15;
    const int col = db * 32 + 16 * g + 4 * (s4 & 3);
    const int ch = col >> 3, half = (col >> 2) & 1;
    const int r0 = k16 * 16 + 4 * hh + (s4 >> 2), r1 = r0 + 8;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(t + r0 * ROWB + pos(r0, ch) * 16 + half * 8));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(t + r1 * ROWB + pos(r1, ch) * 16 + half * 8));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return make_uint4(a.x, a.y, b.x, b.y);
  }
  // Direct-to-LDS load of 1 KiB block `blk` of a tile whose first row is
  // `row0` of `src` (rows past `n_rows` re-read the last row).
  __device__ static void load_block(const uint8_t* src, int64_t row0, int n_rows, int r_base, uint8_t* dst, int blk,
                                    int lane) {
    const int r = blk * RPK + lane / CH;
    const int row = min(r_base + r, n_rows - 1);
    __builtin_amdgcn_global_load_lds(src + (row0 + row) * ROWB + pos(r, lane % CH) * 16,
                                     (lds_void_t*)(dst + blk * 1024), 16, 0, 0);
  }
};

__device__ __forceinline__ uint4 pack8(f16_t t, const f32x16_t& v, int b) {
  return make_uint4(pack2(t, v[b + 0], v[b + 1]), pack2(t, v[b + 2], v[b + 3]), pack2(t, v[b + 4], v[b + 5]),
                    pack2(t, v[b + 6], v[b + 7]));
}
__device__ __forceinline__ uint4 pack8(bf16_t t, const f32x16_t& v, int b) {
  return make_uint4(pack2(t, v[b + 0], v[b + 1]), pack2(t, v[b + 2], v[b + 3]), pack2(t, v[b + 4], v[b + 5]),
                    pack2(t, v[b + 6], v[b + 7]));
}

// The rows one work item sees: its sequence's queries and keys for one
// head (dense batches: the whole head).
struct SeqView {
  int64_t q_row0, k_row0;  // first row of the sequence in the [.., N, d] arrays
  int q_len, k_len;
};

// The rows of the tile in slot t of a variable-length batch (R-row tiles of
// the keys when by_keys, else of the queries; sched::slot_tile), its index
// within its sequence in `local`; false for a slot no tile owns.
template <int R, bool BY_KEYS>
__device__ __forceinline__ bool varlen_tile(const BwdParams& p, int head, int t, SeqView& v, int& local) {
  sched::SlotTile st;
  if (!sched::find_tile<R>(BY_KEYS ? p.cu_k : p.cu_q, p.B, BY_KEYS ? p.Nk : p.Nq, BY_KEYS ? p.cu_q : p.cu_k,
                           BY_KEYS ? p.Nq : p.Nk, t, st))
    return false;
  const int qa = BY_KEYS ? st.oa : st.a, qb = BY_KEYS ? st.oe : st.e;
  const int ka = BY_KEYS ? st.a : st.oa, kb = BY_KEYS ? st.e : st.oe;
  v.q_row0 = (int64_t)head * p.Nq + qa;
  v.k_row0 = (int64_t)head * p.Nk + ka;
  v.q_len = qb - qa;
  v.k_len = kb - ka;
  local = st.j;
  return true;
}

__device__ __forceinline__ SeqView dense_view(const BwdParams& p, int head) {
  return SeqView{(int64_t)head * p.Nq, (int64_t)head * p.Nk, p.Nq, p.Nk};
}

// Store a 32-row block of a transposed accumulator: lane l owns output row
// `row` (a key or a query) and columns 32 db + 8 g + 4 (l / 32) + (0..3).
template <typename TT, int DB>
__device__ __forceinline__ void store_rows(uint16_t* dst_row, const f32x16_t (&acc)[DB], float mul, int hh) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(uint2*)(dst_row + db * 32 + 8 * g + 4 * hh) =
          make_uint2(pack2(TT{}, acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul),
                     pack2(TT{}, acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul));
}

// ---------------------------------------------------------------------------
// delta_i = sum_c dO_ic O_ic: D/8 threads per row, 8 values each.
// ---------------------------------------------------------------------------
constexpr int kDeltaThreads = 256;

template <typename TT, int D>
__global__ void __launch_bounds__(kDeltaThreads) attn_bwd_delta_kernel(BwdParams p, int64_t rows) {
  constexpr int TPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (kDeltaThreads / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const uint4 a = *(const uint4*)((const uint16_t*)p.o + row * D + part * 8);
    const uint4 b = *(const uint4*)((const uint16_t*)p.dout + row * D + part * 8);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t x = unpack2(TT{}, aw[i]), y = unpack2(TT{}, bw[i]);
      acc = __builtin_fmaf(x[0], y[0], acc);
      acc = __builtin_fmaf(x[1], y[1], acc);
    }
  }
#pragma unroll
  for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s, TPR);
  if (row < rows && part == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV.
// ---------------------------------------------------------------------------
template <typename TT, int D, int NW, int WPE, int NS, bool CAUSAL>
__device__ __forceinline__ void dkdv_body(const BwdParams& p, const SeqView sv, const int kt) {
  using T = Tile<D>;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int TILEB = 32 * T::ROWB;            // one 32-row tile of Q or dO
  constexpr int BLK = TILEB / 1024;              // 1 KiB loads per tile
  constexpr int STAGE = 2 * TILEB + 256;         // Q, dO, then lse[32] and delta[32]
  constexpr int LPT = 2 * BLK / NW + 1;          // load instructions per wave per stage
  static_assert((2 * BLK) % NW == 0, "each wave issues the same number of loads");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int64_t q_row0 = sv.q_row0, k_row0 = sv.k_row0;
  const int q_len = sv.q_len, k_len = sv.k_len;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int k0 = kt * 32 * NW, kw0 = k0 + 32 * wv;
  const int my_key = kw0 + c;
  const float cs = p.c;

  // this wave's 32 keys of K as B operands in registers (column = key,
  // k-slice of d); the workgroup's V rows in LDS after the ring, read as B
  // operands of dP (registers are the limit at two waves per SIMD)
  uint8_t* const ldsV = lds + NS * STAGE;
  {
    constexpr int VBLK = 32 * NW * T::ROWB / 1024;
#pragma unroll
    for (int i = 0; i < VBLK / NW; ++i)
      T::load_block((const uint8_t*)p.v, k_row0, k_len, k0, ldsV, wv * (VBLK / NW) + i, lane);
  }
  uint4 kf[KS];
  {
    const int key = min(my_key, k_len - 1);
    const uint16_t* kr = (const uint16_t*)p.k + (k_row0 + key) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const uint4*)(kr + ks * 16);
  }
  f32x16_t dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16_t{};
    dv[db] = f32x16_t{};
  }

  // query blocks of 32 rows: causal starts at the block of the workgroup's
  // first key (for the later waves the first blocks are fully masked: they
  // run them rather than branch around them, which costs the compiler
  // dozens of registers)
  const int n_qb = (q_len + 31) / 32;
  const int qb0 = CAUSAL ? min(k0 / 32, n_qb) : 0;
  const int n_steps = n_qb - qb0;

  auto load_stage = [&](int qb, int slot) {
    uint8_t* st = lds + slot * STAGE;
#pragma unroll
    for (int i = 0; i < 2 * BLK / NW; ++i) {
      const int blk = wv * (2 * BLK / NW) + i;  // blocks 0..BLK-1: Q, BLK..: dO
      if (blk < BLK) T::load_block((const uint8_t*)p.q, q_row0, q_len, qb * 32, st, blk, lane);
      else T::load_block((const uint8_t*)p.dout, q_row0, q_len, qb * 32, st + TILEB, blk - BLK, lane);
    }
    // lse and delta: 64 floats, 16 per wave (4-byte direct-to-LDS loads)
    const int idx = 16 * (wv & 3) + (lane & 15);
    const int q = min(qb * 32 + (idx & 31), q_len - 1);
    const float* src = (idx < 32 ? p.lse : p.delta) + q_row0 + q;
    if (wv < 4 && lane < 16)
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(st + 2 * TILEB + 64 * (wv & 3)), 4, 0, 0);
  };
  static_assert(NW == 4, "the four waves load 16 of the 64 lse and delta values each");

#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_steps) load_stage(qb0 + j, j);
  int slot = 0;
  for (int it = 0; it < n_steps; ++it) {
    const int qb = qb0 + it;
    if (it + NS - 2 < n_steps) bwd_wait_vm<(NS - 2) * LPT>();
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // non-causal: the stage loads go out after the S and dP chain, which then
    // starts at once after the barrier (+2 % at d = 128, +4 % at d = 256;
    // causal launches lose as much and issue them first)
    const bool refill = it + NS - 1 < n_steps;
    if (CAUSAL && refill) load_stage(qb + NS - 1, slot == 0 ? NS - 1 : slot - 1);
    {
      const uint8_t* tq = lds + slot * STAGE;
      const uint8_t* tdo = tq + TILEB;
      const float* tl = (const float*)(tq + 2 * TILEB);
      // S = Q K^T and dP = dO V^T: column = this lane's key, rows = queries
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(TT{}, T::rows_frag(tq, c, ks, hh), kf[ks], s);
        dp = mfma32(TT{}, T::rows_frag(tdo, c, ks, hh), T::rows_frag(ldsV, 32 * wv + c, ks, hh), dp);
      }
      if (!CAUSAL && refill) load_stage(qb + NS - 1, slot == 0 ? NS - 1 : slot - 1);
      const bool masked = (CAUSAL && qb * 32 < kw0 + 31) || qb * 32 + 32 > q_len;
      // element (g, j) is query q = qb*32 + 4 hh + 8 g + j: it exists iff
      // 8 g + j < q_lim and sees this lane's key iff 8 g + j >= key_rel
      // (comparisons against constants, nothing kept live across blocks)
      const int q_lim = q_len - qb * 32 - 4 * hh;
      const int key_rel = my_key - qb * 32 - 4 * hh;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 l4 = *(const float4*)(tl + 8 * g + 4 * hh);
        const float4 d4 = *(const float4*)(tl + 32 + 8 * g + 4 * hh);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * g + j;
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], cs, -lv[j] * kLog2e));
          if (masked && (8 * g + j >= q_lim || (CAUSAL && 8 * g + j < key_rel))) pv = 0.f;
          s[i] = pv;
          dp[i] = pv * (dp[i] - dl[j]);
        }
      }
      uint4 pp[2], dsp[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        pp[h2] = pack8(TT{}, s, 8 * h2);
        dsp[h2] = pack8(TT{}, dp, 8 * h2);
      }
      // dV^T += dO^T P^T, dK^T += Q^T dS^T over the block's 32 queries
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = mfma32(TT{}, T::cols_frag(tdo, db, h2, lane), pp[h2], dv[db]);
          dk[db] = mfma32(TT{}, T::cols_frag(tq, db, h2, lane), dsp[h2], dk[db]);
        }
    }
    slot = (slot + 1 == NS) ? 0 : slot + 1;
  }

  if (my_key < k_len) {
    store_rows<TT, DB>((uint16_t*)p.dk + (k_row0 + my_key) * D, dk, p.scale, hh);
    store_rows<TT, DB>((uint16_t*)p.dv + (k_row0 + my_key) * D, dv, 1.f, hh);
  }
}

// The key tiles of one head run on one XCD (shared L2 copy of the head's Q
// and dO).  Causal: key tile kt sees the queries from kt*32*NW on, so the
// work falls with kt; a workgroup takes tiles j and T-1-j of one head in
// turn (p.n_work counts the pairs), so that all do the same work.
// Variable-length batches: a head's key tiles are numbered by slot
// (sched::slot_tile; p.tiles_per_head bounds the slots, surplus workgroups
// exit).
template <typename TT, int D, int NW, int WPE, int NS, bool CAUSAL, bool VARLEN>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(WPE, WPE)))
attn_bwd_dkdv_kernel(BwdParams p) {
  const int w = xcd_remap(blockIdx.x, p.n_work);
  if constexpr (VARLEN) {
    const int head = w / p.tiles_per_head;
    SeqView sv;
    int kt;
    if (varlen_tile<32 * NW, true>(p, head, w - head * p.tiles_per_head, sv, kt))
      dkdv_body<TT, D, NW, WPE, NS, CAUSAL>(p, sv, kt);
  } else if constexpr (CAUSAL) {
    const int T = p.tiles_per_head, half = (T + 1) / 2;
    const int head = w / half, j = w - head * half;
    dkdv_body<TT, D, NW, WPE, NS, CAUSAL>(p, dense_view(p, head), j);
    if (T - 1 - j != j) {
      __syncthreads();
      dkdv_body<TT, D, NW, WPE, NS, CAUSAL>(p, dense_view(p, head), T - 1 - j);
    }
  } else {
    const int head = w / p.tiles_per_head;
    dkdv_body<TT, D, NW, WPE, NS, CAUSAL>(p, dense_view(p, head), w - head * p.tiles_per_head);
  }
}

// ---------------------------------------------------------------------------
// dQ.
// ---------------------------------------------------------------------------
template <typename TT, int D, int BC, int NW, int WPE, int NS, bool CAUSAL>
__device__ __forceinline__ void dq_body(const BwdParams& p, const SeqView sv, const int qt) {
  using T = Tile<D>;
  constexpr int KS = D / 16, DB = D / 32, MB = BC / 32;
  constexpr int TILEB = BC * T::ROWB;
  constexpr int BLK = TILEB / 1024;
  constexpr int STAGE = 2 * TILEB;               // K then V
  constexpr int LPT = 2 * BLK / NW;
  static_assert((2 * BLK) % NW == 0, "each wave issues the same number of loads");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int64_t q_row0 = sv.q_row0, k_row0 = sv.k_row0;
  const int q_len = sv.q_len, k_len = sv.k_len;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int q0 = qt * 32 * NW, qw0 = q0 + 32 * wv;
  const int my_q = qw0 + c;
  const float cs = p.c;

  uint4 qf[KS], df[KS];
  float lse2 = 0.f, dl = 0.f;
  {
    const int q = min(my_q, q_len - 1);
    const uint16_t* qr = (const uint16_t*)p.q + (q_row0 + q) * D + 8 * hh;
    const uint16_t* dr = (const uint16_t*)p.dout + (q_row0 + q) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *(const uint4*)(qr + ks * 16);
      df[ks] = *(const uint4*)(dr + ks * 16);
    }
    lse2 = p.lse[q_row0 + q] * kLog2e;
    dl = p.delta[q_row0 + q];
  }
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};

  int n_kt = (k_len + BC - 1) / BC, wave_kt = n_kt;
  if (CAUSAL) {
    const int last_wg = min(q0 + 32 * NW, q_len) - 1;  // the workgroup's last query
    n_kt = last_wg < 0 ? 0 : min(n_kt, last_wg / BC + 1);
    const int last_w = min(qw0 + 31, q_len - 1);
    wave_kt = last_w < 0 ? 0 : min(n_kt, last_w / BC + 1);
  }
  if (qw0 >= q_len) wave_kt = 0;

  auto load_stage = [&](int kt, int slot) {
    uint8_t* st = lds + slot * STAGE;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int blk = wv * LPT + i;
      if (blk < BLK) T::load_block((const uint8_t*)p.k, k_row0, k_len, kt * BC, st, blk, lane);
      else T::load_block((const uint8_t*)p.v, k_row0, k_len, kt * BC, st + TILEB, blk - BLK, lane);
    }
  };

#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_kt) load_stage(j, j);
  int slot = 0;
  for (int kt = 0; kt < n_kt; ++kt) {
    if (kt + NS - 2 < n_kt) bwd_wait_vm<(NS - 2) * LPT>();
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // non-causal: a live wave issues the stage loads after its S and dP
    // chain (as in the dK/dV kernel)
    const bool refill = kt + NS - 1 < n_kt;
    if ((CAUSAL || kt >= wave_kt) && refill) load_stage(kt + NS - 1, slot == 0 ? NS - 1 : slot - 1);
    if (kt < wave_kt) {
      const uint8_t* tk = lds + slot * STAGE;
      const uint8_t* tv = tk + TILEB;
      // S^T = K Q^T, dP^T = V dO^T: column = this lane's query, rows = keys
      f32x16_t s[MB], dp[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        s[mb] = f32x16_t{};
        dp[mb] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s[mb] = mfma32(TT{}, T::rows_frag(tk, mb * 32 + c, ks, hh), qf[ks], s[mb]);
          dp[mb] = mfma32(TT{}, T::rows_frag(tv, mb * 32 + c, ks, hh), df[ks], dp[mb]);
        }
      }
      if (!CAUSAL && refill) load_stage(kt + NS - 1, slot == 0 ? NS - 1 : slot - 1);
      const bool masked = (CAUSAL && kt * BC + BC - 1 > qw0) || kt * BC + BC > k_len;
      // element (mb, i) is key kt*BC + 4 hh + e with e = 32 mb + 8 (i/4) + i%4:
      // it exists iff e < k_lim and is visible to this lane's query iff e <= q_rel
      const int k_lim = k_len - kt * BC - 4 * hh;
      const int q_rel = my_q - kt * BC - 4 * hh;
      uint4 dsp[MB][2];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][i], cs, -lse2));
          const int e = 32 * mb + 8 * (i >> 2) + (i & 3);
          if (masked && (e >= k_lim || (CAUSAL && e > q_rel))) pv = 0.f;
          dp[mb][i] = pv * (dp[mb][i] - dl);
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) dsp[mb][h2] = pack8(TT{}, dp[mb], 8 * h2);
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int k16 = 0; k16 < 2 * MB; ++k16)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = mfma32(TT{}, T::cols_frag(tk, db, k16, lane), dsp[k16 >> 1][k16 & 1], acc[db]);
    }
    slot = (slot + 1 == NS) ? 0 : slot + 1;
  }
  if (my_q < q_len) store_rows<TT, DB>((uint16_t*)p.dq + (q_row0 + my_q) * D, acc, p.scale, hh);
}

// Causal: query tile qt sees the keys up to its last row; a workgroup takes
// tiles T-1-j (the heaviest) and j in turn (p.n_work counts the pairs).
template <typename TT, int D, int BC, int NW, int WPE, int NS, bool CAUSAL, bool VARLEN>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(WPE, WPE)))
attn_bwd_dq_kernel(BwdParams p) {
  const int w = xcd_remap(blockIdx.x, p.n_work);
  if constexpr (VARLEN) {
    const int head = w / p.tiles_per_head;
    SeqView sv;
    int qt;
    if (varlen_tile<32 * NW, false>(p, head, w - head * p.tiles_per_head, sv, qt))
      dq_body<TT, D, BC, NW, WPE, NS, CAUSAL>(p, sv, qt);
  } else if constexpr (CAUSAL) {
    const int T = p.tiles_per_head, half = (T + 1) / 2;
    const int head = w / half, j = w - head * half;
    dq_body<TT, D, BC, NW, WPE, NS, CAUSAL>(p, dense_view(p, head), T - 1 - j);
    if (T - 1 - j != j) {
      __syncthreads();
      dq_body<TT, D, BC, NW, WPE, NS, CAUSAL>(p, dense_view(p, head), j);
    }
  } else {
    const int head = w / p.tiles_per_head;
    dq_body<TT, D, BC, NW, WPE, NS, CAUSAL>(p, dense_view(p, head), w - head * p.tiles_per_head);
  }
}

// ---------------------------------------------------------------------------
// Launch configurations.
// ---------------------------------------------------------------------------
// dK/dV: NW waves of 32 keys, WPE waves per SIMD, an NS-slot ring of
// 32-query blocks.  At d = 128 a wave holds K (32 registers) and the dK, dV
// accumulators (128); V sits in LDS.  Measured at d = 128: with V in
// registers too, two waves per SIMD spill ~20 values (still 14 % faster
// than one wave per SIMD), and V in LDS removes the spills (+14 %); the
// 2-slot ring keeps two workgroups within a CU's LDS.  dQ: 64-key tiles in a
// 2-slot ring, two waves per SIMD.
template <int D>
struct BwdCfg {
  static constexpr int NW = 4, WPE = 2, NS = 2;
  static constexpr int DQ_BC = 64, DQ_NW = 4, DQ_WPE = 2, DQ_NS = 2;
};
// d = 256: the dK and dV accumulators alone take 256 registers per lane, so
// one wave per SIMD (512 registers, accumulators in AGPRs); LDS 128.5 KiB
// (dK/dV: two 32-row Q/dO stages and 128 V rows) and 128 KiB (dQ: four
// slots of 32 keys; with one wave per SIMD the shorter steps and deeper
// ring measured 5.80 -> 5.54 ms for the whole backward at B1 H16 N8192,
// against two slots of 64 keys; at two waves per SIMD, d = 64 and 128, they
// measured 1-3 % slower).
template <>
struct BwdCfg<256> {
  static constexpr int NW = 4, WPE = 1, NS = 2;
  static constexpr int DQ_BC = 32, DQ_NW = 4, DQ_WPE = 1, DQ_NS = 4;
};

template <typename TT, int D, bool CAUSAL, bool VARLEN>
hipError_t launch_bwd_t(BwdParams p, hipStream_t st) {
  const int64_t heads = VARLEN ? p.H : (int64_t)p.B * p.H;  // varlen arrays are [H, T, d]
  const int64_t rows = heads * p.Nq;
  if (rows > 0) {
    constexpr int RPB = kDeltaThreads / (D / 8);
    hipLaunchKernelGGL((attn_bwd_delta_kernel<TT, D>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                       dim3(kDeltaThreads), 0, st, p, rows);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if (p.Nk > 0) {
    using C = BwdCfg<D>;
    constexpr int STAGE = 2 * 32 * D * 2 + 256;
    constexpr int lds = C::NS * STAGE + 32 * C::NW * D * 2;
    auto kern = attn_bwd_dkdv_kernel<TT, D, C::NW, C::WPE, C::NS, CAUSAL, VARLEN>;
    if (hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        e != hipSuccess)
      return e;
    BwdParams pk = p;
    pk.tiles_per_head = (p.Nk + 32 * C::NW - 1) / (32 * C::NW) + (VARLEN ? p.B : 0);
    pk.n_work = (int)heads * (CAUSAL && !VARLEN ? (pk.tiles_per_head + 1) / 2 : pk.tiles_per_head);
    hipLaunchKernelGGL(kern, dim3(pk.n_work), dim3(C::NW * 64), lds, st, pk);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if (p.Nq > 0) {
    using C = BwdCfg<D>;
    constexpr int lds = C::DQ_NS * 2 * C::DQ_BC * D * 2;
    auto kern = attn_bwd_dq_kernel<TT, D, C::DQ_BC, C::DQ_NW, C::DQ_WPE, C::DQ_NS, CAUSAL, VARLEN>;
    if (hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        e != hipSuccess)
      return e;
    BwdParams pq = p;
    pq.tiles_per_head = (p.Nq + 32 * C::DQ_NW - 1) / (32 * C::DQ_NW) + (VARLEN ? p.B : 0);
    pq.n_work = (int)heads * (CAUSAL && !VARLEN ? (pq.tiles_per_head + 1) / 2 : pq.tiles_per_head);
    hipLaunchKernelGGL(kern, dim3(pq.n_work), dim3(C::DQ_NW * 64), lds, st, pq);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TT, int D>
hipError_t launch_bwd_cv(bool causal, bool varlen, const BwdParams& p, hipStream_t st) {
  if (varlen) return causal ? launch_bwd_t<TT, D, true, true>(p, st) : launch_bwd_t<TT, D, false, true>(p, st);
  return causal ? launch_bwd_t<TT, D, true, false>(p, st) : launch_bwd_t<TT, D, false, false>(p, st);
}

template <typename TT>
hipError_t launch_bwd_d(int d, bool causal, bool varlen, const BwdParams& p, hipStream_t st) {
  switch (d) {
    case 64: return launch_bwd_cv<TT, 64>(causal, varlen, p, st);
    case 128: return launch_bwd_cv<TT, 128>(causal, varlen, p, st);
    case 256: return launch_bwd_cv<TT, 256>(causal, varlen, p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int bwd_key_block(int d) {
  return 32 * (d == 64 ? BwdCfg<64>::NW : d == 128 ? BwdCfg<128>::NW : BwdCfg<256>::NW);
}
int bwd_query_block(int d) {
  return 32 * (d == 64 ? BwdCfg<64>::DQ_NW : d == 128 ? BwdCfg<128>::DQ_NW : BwdCfg<256>::DQ_NW);
}

hipError_t launch_bwd(int dtype, int d, bool causal, bool varlen, BwdParams p, hipStream_t st) {
  return dtype == 0 ? launch_bwd_d<f16_t>(d, causal, varlen, p, st) : launch_bwd_d<bf16_t>(d, causal, varlen, p, st);
}

}  // namespace attn
