// Backward pass of attention on fp8 operands, gfx950 (CDNA4) fp8 MFMA.
//
// "Flash Attention 3：让 GPU 跑满的注意力计算", §4.1.2 gives the forward pass
// E4M3 and back-propagation E5M2 (more range, less precision); it prints no
// algorithm.  The gradients are those of the attention of the fp8 forward's
// operands (the chain rule, as in attn_bwd.hip):
//
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - delta),  delta_i = dO_i . O_i,
//   dQ = scale dS K,  dK = scale dS^T Q,
//
// with all five products on the 32x32x64 fp8 MFMA (fp32 accumulation):
// Q, K, V are the forward's e4m3 codes with their per-128-row-tile scales;
// dO is quantised to e5m2 with one scale per 128-row tile; P is rounded to
// e4m3 and dS to e5m2.  The per-tile scale of the operand a product sums
// over is folded into the factor rounded in the kernel (as the forward folds
// the V tile's scale into P), so no product needs a per-tile correction:
//
//   dV = max s_do 2^-8 sum_q P8 do8,    P8  = e4m3(2^8 P s_do(q) / max s_do)
//   dK = scale max s_q sum_q dSq q8,    dSq = e5m2(dS s_q(q) / max s_q)
//   dQ = scale max s_k sum_k dSk k8,    dSk = e5m2(dS s_k(k) / max s_k)
//
// Three kernels, like the 16-bit backward: a pre-processing pass (delta from
// O and dO, and dO's e5m2 codes and scales), a key-stationary dK/dV pass
// (each wave 32 keys with its K and V rows in registers; 64-row blocks of Q
// and dO stream through an LDS ring) and a query-stationary dQ pass (each
// wave 32 queries with Q and dO in registers; 64-key blocks of K and V
// stream).  The 64-row blocks make the transposed products (dO^T P^T,
// Q^T dS^T, K^T dS^T) one MFMA k-step of 64 queries (keys).
//
// Operand layouts follow the e4m3 forward: an MFMA operand "by rows" gives
// lane (c, h) row c and bytes [64 ks + 32 h, +32) of its 128-byte row; the
// accumulator of a 32x32 product gives lane (c, h) column c and rows
// 8 (i / 4) + 4 h + i % 4, i = 0..15, and its 32 values of two such blocks
// (rows 0..31 and 32..63) are, in that order, the B operand of the product
// that sums over those 64 rows; the A operand of that product (the
// transposed tile) comes from ds_read_b64_tr_b8 reads of the row-major tile
// with its k-index in the same order.  Each tile read both ways is stored
// twice in LDS, once per swizzle (the row reads and the transposing reads
// are conflict-free under different chunk permutations).
#include <type_traits>

#include "attn_device.h"
#include "attn_params.h"

namespace attn {
namespace {

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kD = 128;            // head dimension
constexpr int kRowB = kD;          // bytes per row of codes
constexpr int kScaleRows = 128;    // rows per scale entry
constexpr int kBlk = 64;           // rows of a streamed block
constexpr int kBlkB = kBlk * kRowB;  // 8 KiB
constexpr float kE5m2Max = 57344.f;
constexpr float kF32Tiny = 0x1p-149f;
constexpr float kPScale = 256.f;
constexpr int kFmtE4m3 = 0, kFmtE5m2 = 1;  // MFMA operand formats (f8f6f4 selectors)

// 32x32x64 fp8 MFMA with operand formats FA (A) and FB (B).
template <int FA, int FB>
__device__ __forceinline__ f32x16_t mfma8(const uint4& a0, const uint4& a1, const uint4& b0, const uint4& b1,
                                          const f32x16_t& c) {
  i32x8_t a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  i32x8_t b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// Chunk permutations of 128-byte rows (8 chunks of 16 bytes), as in the
// e4m3 forward: rows8 for reads by rows (16 lanes, 16 rows, one chunk),
// tr8 for the transposing reads (8 rows x 2 chunks per 32 lanes).
__device__ __forceinline__ int rows8(int r, int ch) { return ch ^ ((r >> 1) & 7); }
__device__ __forceinline__ int tr8(int r, int ch) { return ch ^ (((r >> 1) & 1) << 1) ^ (((r >> 3) & 1) << 2); }

// Operand by rows: row `row` of tile t (rows8 layout), k-step ks, lane half h.
__device__ __forceinline__ void row_frag(const uint8_t* t, int row, int ks, int h, uint4& f0, uint4& f1) {
  const int ch = 4 * ks + 2 * h;
  f0 = *(const uint4*)(t + row * kRowB + rows8(row, ch) * 16);
  f1 = *(const uint4*)(t + row * kRowB + rows8(row, ch + 1) * 16);
}

// Transposed operand of a 64-row tile (tr8 layout): output block db (32
// columns of the tile), k-index 32 h + j of lane half h = tile row
// 32 (j / 16) + 8 ((j % 16) / 4) + 4 h + j % 4.  In 16-lane group G, source
// lane s reads row 8 m' + ... : four reads m = 0..3 give k-indices 8m..8m+7
// (bytes of the 8-byte pieces read by lanes 2j + s / 8).
struct TrOffsets {
  uint32_t off[kD / 32];
  __device__ explicit TrOffsets(int lane) {
    const int hh = lane >> 5, G = lane >> 4, s16 = lane & 15, b = s16 >> 1;
    const int lr = 8 * (b >> 2) + 4 * hh + (b & 3);  // the lane's row within 16
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
      off[db] = (uint32_t)(lr * kRowB + tr8(lr, 2 * db + (G & 1)) * 16 + 8 * (s16 & 1));
  }
};
__device__ __forceinline__ void tr_frag(const uint8_t* t, uint32_t off, uint4& f0, uint4& f1) {
  uint32_t w[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int rstep = 32 * (m >> 1) + 16 * (m & 1);  // a multiple of 16 rows
    const i32x2_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2_t*)(t + off + rstep * kRowB));
    w[2 * m] = (uint32_t)x[0];
    w[2 * m + 1] = (uint32_t)x[1];
  }
  f0 = make_uint4(w[0], w[1], w[2], w[3]);
  f1 = make_uint4(w[4], w[5], w[6], w[7]);
}

// Sixteen fp32 values -> 16 e4m3 / e5m2 codes (round to nearest even; e5m2
// clamped to +-57344 first).  Each first conversion's "old" operand (whose
// upper half it keeps, and the second conversion overwrites) is its first
// value's bits, so no register has to be zeroed for it.
__device__ __forceinline__ uint4 pack16_e4m3(const f32x16_t& v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i], v[4 * i + 1], __builtin_bit_cast(int, v[4 * i]), false);
    w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i + 2], v[4 * i + 3], x, true);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ float clamp_e5m2(float x) { return __builtin_amdgcn_fmed3f(x, -kE5m2Max, kE5m2Max); }
__device__ __forceinline__ uint4 pack16_e5m2(const f32x16_t& v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = clamp_e5m2(v[4 * i]);
    int x = __builtin_amdgcn_cvt_pk_bf8_f32(a, clamp_e5m2(v[4 * i + 1]), __builtin_bit_cast(int, a), false);
    w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(clamp_e5m2(v[4 * i + 2]), clamp_e5m2(v[4 * i + 3]), x, true);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Largest of the n scale entries at s (every lane of the wave gets it).
__device__ __forceinline__ float scale_max(const float* s, int n, int lane) {
  float m = 0.f;
  for (int j = lane; j < n; j += 64) m = fmaxf(m, s[j]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k));
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, m)));
}

// Byte offsets (within a 1 KiB block of 8 rows) that lane `lane` fetches
// for a direct-to-LDS tile load: the lane writes physical chunk lane % 8 of
// row lane / 8 and so fetches the logical chunk stored there.  The chunk
// permutations read bits 1..3 of the row, and bit 3 is the parity of the
// block: entry par serves the blocks of that parity.
struct TileLane {
  uint32_t vo[2];
  __device__ TileLane(int lane, bool tr) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int r = 8 * par + (lane >> 3);
      const int ch = tr ? tr8(r, lane & 7) : rows8(r, lane & 7);
      vo[par] = (uint32_t)((lane >> 3) * kRowB + ch * 16);
    }
  }
};

// 1 / x (correctly rounded), or 0 for x = 0 (a head whose scales are all 0
// has an all-zero operand; its fold ratios are then 0).
__device__ __forceinline__ float recip_or_zero(float x) { return x > 0.f ? 1.0f / x : 0.f; }

// Direct-to-LDS load of a 64-row tile (8 KiB) by one wave: rows r0 ..
// r0 + 63 of the rows at `base` (n_rows of them, r0 < n_rows) go to dst
// with their chunks permuted (rows8, or tr8 if tr).  The rows come through a
// buffer resource based at row r0, so a full tile costs no vector
// instructions; a tile that runs past n_rows clamps each lane's row to the
// last one, so no read goes out of range.
__device__ __forceinline__ void load_tile64(const uint8_t* base, int r0, int n_rows, uint8_t* dst,
                                            const TileLane& tl, bool tr, int lane) {
  const int rows = min(kBlk, n_rows - r0);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)r0 * kRowB), 0, rows * kRowB, kBufferFlags);
  if (rows == kBlk) {
#pragma unroll
    for (int b = 0; b < 8; ++b)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + b * 1024), 16, tl.vo[b & 1],
                                               (uint32_t)(b * 1024), 0, 0);
  } else {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int r = 8 * b + (lane >> 3);
      const int ch = tr ? tr8(r, lane & 7) : rows8(r, lane & 7);
      const uint32_t off = (uint32_t)(min(r, rows - 1) * kRowB + ch * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + b * 1024), 16, off, 0, 0, 0);
    }
  }
}

// Direct-to-LDS load of 64 floats (rows r0 .. r0 + 63 of the n_rows at
// base; lanes past the end re-read the last one) to dst.
__device__ __forceinline__ void load_row_floats(const float* base, int r0, int n_rows, uint8_t* dst, int lane) {
  const int rows = min(kBlk, n_rows - r0);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + r0), 0, rows * 4, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 4, (uint32_t)(min(lane, rows - 1) * 4), 0, 0, 0);
}

// Store a 32-row block of a transposed accumulator: lane (c, h) owns output
// row `dst_row` and columns 32 db + 8 g + 4 h + (0..3).
__device__ __forceinline__ void store_rows_bf16(uint16_t* dst_row, const f32x16_t (&acc)[kD / 32], float mul,
                                                int hh) {
#pragma unroll
  for (int db = 0; db < kD / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(uint2*)(dst_row + db * 32 + 8 * g + 4 * hh) =
          make_uint2(pack2(bf16_t{}, acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul),
                     pack2(bf16_t{}, acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul));
}

// ---------------------------------------------------------------------------
// Pre-processing: one workgroup per (b*h, 128-row tile) of dO and O.
// dO: s = amax(dO tile) / 57344 (1 if the tile is all zero, at least
// 2^-149) and codes e5m2(dO / s).  Row statistics for the other kernels, in
// the three planes of the stats workspace: L2_i = lse_i log2(e), delta_i =
// sum_c dO_ic O_ic in fp32, and delta_i f_q with f_q = s_q(tile) / max s_q
// (the dK pass multiplies P (dP - delta) by f_q; folding it into delta and
// into dP's scale saves a multiplication per element).  f_q is formed as
// s_q(tile) * recip_or_zero(max s_q) here and in the dK pass, so both take
// the same value.  Two threads per row, 64 values each.
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 256;

__global__ void __launch_bounds__(kPrepThreads) bwd8_prep_kernel(Bwd8Params p) {
  __shared__ float red[kPrepThreads / 64];
  const int nt = (p.Nq + kScaleRows - 1) / kScaleRows;
  const int bh = blockIdx.x / nt, tile = blockIdx.x - bh * nt;
  const int row = tile * kScaleRows + (threadIdx.x >> 1), half = threadIdx.x & 1;
  const bool live = row < p.Nq;
  const int64_t base = ((int64_t)bh * p.Nq + (live ? row : 0)) * kD + half * 64;
  const float* sq = p.q_scale + (int64_t)bh * nt;
  float sq_max = 0.f;
  for (int j = threadIdx.x & 63; j < nt; j += 64) sq_max = fmaxf(sq_max, sq[j]);
  float v[64];
  float dsum = 0.f, amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint4 a = zero4(), b = zero4();
    if (live) {
      a = *(const uint4*)((const uint16_t*)p.dout + base + 8 * i);
      b = *(const uint4*)((const uint16_t*)p.o + base + 8 * i);
    }
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x2_t x = unpack2(bf16_t{}, aw[j]), y = unpack2(bf16_t{}, bw[j]);
      v[8 * i + 2 * j] = x[0];
      v[8 * i + 2 * j + 1] = x[1];
      dsum = __builtin_fmaf(x[0], y[0], dsum);
      dsum = __builtin_fmaf(x[1], y[1], dsum);
      amax = fmaxf(amax, fmaxf(fabsf(x[0]), fabsf(x[1])));
    }
  }
  dsum += __shfl_xor(dsum, 1);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, s));
    sq_max = fmaxf(sq_max, __shfl_xor(sq_max, s));
  }
  if (live && half == 0) {
    const int64_t r = (int64_t)bh * p.Nq + row;
    p.stats[r] = p.lse[r] * kLog2e;
    const int64_t plane = (int64_t)p.B * p.H * p.Nq;
    p.stats[plane + r] = dsum;
    p.stats[2 * plane + r] = dsum * (sq[tile] * recip_or_zero(sq_max));
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  float tmax = red[0];
#pragma unroll
  for (int i = 1; i < kPrepThreads / 64; ++i) tmax = fmaxf(tmax, red[i]);
  const float s = tmax > 0.f ? fmaxf(tmax / kE5m2Max, kF32Tiny) : 1.0f;
  if (threadIdx.x == 0) p.do_scale[(int64_t)bh * nt + tile] = s;
  if (!live) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // 16 values -> 16 codes per iteration
    f32x16_t z;
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = v[16 * i + j] / s;  // correctly rounded fp32 division
    *(uint4*)(p.do8 + base + 16 * i) = pack16_e5m2(z);
  }
}

// ---------------------------------------------------------------------------
// dK, dV: a workgroup of 4 waves owns 128 keys (one K/V scale tile) of one
// head; 64-row blocks of Q and dO (each stored twice: rows8 and tr8), L2 and
// delta f_q stream through a 2-slot LDS ring.  A step handles its
// 64 queries as two 32-row halves (S, dP, then P and dS packed to 8 bits),
// so that only one half's fp32 values are live: with the 128 accumulator
// registers of dK and dV the wave fits in 256 registers, two waves per SIMD.
// Blocks that the causal diagonal or the ends of the sequences cut run the
// masked variant of the element-wise step; the others run it without masks.
// ---------------------------------------------------------------------------
constexpr int kNW = 4;
constexpr int kStage = 4 * kBlkB + 2 * kBlk * 4;  // Q rows8, Q tr8, dO rows8, dO tr8, L2[64], delta f_q[64]

template <bool CAUSAL>
__device__ __forceinline__ void dkdv8_body(const Bwd8Params& p, const int head, const int kt) {
  constexpr int DB = kD / 32;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int Nq = p.Nq, Nk = p.Nk;
  const int nqt = (Nq + kScaleRows - 1) / kScaleRows, nkt = (Nk + kScaleRows - 1) / kScaleRows;
  const int k0 = kt * kScaleRows, my_key = k0 + 32 * wv + c;
  const int kw_last = k0 + 32 * wv + 31;  // the wave's last key
  const int64_t q_row0 = (int64_t)head * Nq, k_row0 = (int64_t)head * Nk;
  const float* sq = p.q_scale + (int64_t)head * nqt;
  const float* sdo = p.do_scale + (int64_t)head * nqt;
  const float* l2g = p.stats;
  const float* dlg = p.stats + 2 * (int64_t)p.B * p.H * Nq;
  const float sq_max = scale_max(sq, nqt, lane), sdo_max = scale_max(sdo, nqt, lane);
  const float rsq = recip_or_zero(sq_max), rsdo = recip_or_zero(sdo_max);
  const float skt = load_uniform(p.k_scale, (int64_t)head * nkt + kt);
  const float svt = load_uniform(p.v_scale, (int64_t)head * nkt + kt);

  // this wave's K and V rows (key my_key) as B operands
  uint4 kf[2][2], vf[2][2];
  {
    const int key = min(my_key, Nk - 1);
    const uint8_t* kr = p.k + (k_row0 + key) * kRowB + 32 * hh;
    const uint8_t* vr = p.v + (k_row0 + key) * kRowB + 32 * hh;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kf[ks][0] = *(const uint4*)(kr + 64 * ks);
      kf[ks][1] = *(const uint4*)(kr + 64 * ks + 16);
      vf[ks][0] = *(const uint4*)(vr + 64 * ks);
      vf[ks][1] = *(const uint4*)(vr + 64 * ks + 16);
    }
  }
  const TrOffsets tro(lane);
  f32x16_t dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16_t{};
    dv[db] = f32x16_t{};
  }

  // query blocks of 64 rows; causal: from the block of the first key on
  const int n_qb = (Nq + kBlk - 1) / kBlk;
  const int qb0 = CAUSAL ? min(k0 / kBlk, n_qb) : 0;
  const int n_steps = n_qb - qb0;

  // wave w loads tile w of a stage: Q rows8, Q tr8, dO rows8, dO tr8; waves
  // 0 and 1 also L2 and delta f_q
  const TileLane tlane(lane, wv & 1);
  const uint8_t* tile_src = (wv < 2 ? p.q : p.do8) + q_row0 * kRowB;
  const float* row_src = (wv == 0 ? l2g : dlg) + q_row0;
  auto load_stage = [&](int qb, uint8_t* st) __attribute__((always_inline)) {
    load_tile64(tile_src, qb * kBlk, Nq, st + wv * kBlkB, tlane, wv & 1, lane);
    if (wv < 2) load_row_floats(row_src, qb * kBlk, Nq, st + 4 * kBlkB + wv * 256, lane);
  };

  // S and dP of query rows 32 nb .. of the block: element i of the
  // accumulators is query row 32 nb + 8 (i/4) + 4 hh + i%4 of the block
  auto sdp = [&](const uint8_t* st, const int nb, f32x16_t& s, f32x16_t& dpa) __attribute__((always_inline)) {
    s = f32x16_t{};
    dpa = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 a0, a1, b0, b1;
      row_frag(st, nb * 32 + c, ks, hh, a0, a1);
      row_frag(st + 2 * kBlkB, nb * 32 + c, ks, hh, b0, b1);
      s = mfma8<kFmtE4m3, kFmtE4m3>(a0, a1, kf[ks][0], kf[ks][1], s);
      dpa = mfma8<kFmtE5m2, kFmtE4m3>(b0, b1, vf[ks][0], vf[ks][1], dpa);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // P and dS of those rows, rounded and packed four rows (one dword) at a
  // time: P8 = e4m3(P fp), dS8 = e5m2(P (dP cdp - delta f_q)).  MASK: the
  // block is cut by the causal diagonal or an end of the sequences.
  auto elementwise = [&](const uint8_t* st, const int qb, const int nb, const f32x16_t& s, const f32x16_t& dpa,
                         const float cs, const float cdp, const float fp, uint4& p8, uint4& d8, auto mask_tag)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const float* tl = (const float*)(st + 4 * kBlkB);
    const float* tdl = tl + kBlk;
    uint32_t pw[4], dw[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = 32 * nb + 8 * g + 4 * hh;
      const float4 L = *(const float4*)(tl + r0);
      const float4 Dl = *(const float4*)(tdl + r0);
      const float Lv[4] = {L.x, L.y, L.z, L.w}, Dv[4] = {Dl.x, Dl.y, Dl.z, Dl.w};
      float xp[4], xs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        float t = __builtin_fmaf(s[i], cs, -Lv[j]);
        if constexpr (MASK) {
          const int q = qb * kBlk + r0 + j;
          const bool ok = (q < Nq) & (my_key < Nk) & (!CAUSAL | (my_key <= q)) & (Lv[j] > -INFINITY);
          t = ok ? t : -INFINITY;
        }
        const float pv = __builtin_amdgcn_exp2f(t);
        xs[j] = clamp_e5m2(pv * __builtin_fmaf(dpa[i], cdp, -Dv[j]));
        xp[j] = pv * fp;
      }
      pw[g] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
          xp[2], xp[3], __builtin_amdgcn_cvt_pk_fp8_f32(xp[0], xp[1], __builtin_bit_cast(int, xp[0]), false), true);
      dw[g] = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(
          xs[2], xs[3], __builtin_amdgcn_cvt_pk_bf8_f32(xs[0], xs[1], __builtin_bit_cast(int, xs[0]), false), true);
      __builtin_amdgcn_sched_barrier(0);
    }
    p8 = make_uint4(pw[0], pw[1], pw[2], pw[3]);
    d8 = make_uint4(dw[0], dw[1], dw[2], dw[3]);
  };

  auto step = [&](const int qb, const uint8_t* st) __attribute__((always_inline)) {
    const int qs = (qb * kBlk) / kScaleRows;  // the block's scale tile
    const float sqb = load_uniform(sq, qs), sdob = load_uniform(sdo, qs);
    const float cs = p.c * sqb * skt;               // S in base 2
    const float cdp = sdob * svt * (sqb * rsq);    // dP, times the dK fold f_q (as delta in the stats)
    const float fp = kPScale * (sdob * rsdo);
    const bool full = (qb + 1) * kBlk <= Nq && kw_last < Nk && (!CAUSAL || qb * kBlk >= kw_last);
    uint4 p8[2], d8[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      f32x16_t sv, dpv;
      sdp(st, nb, sv, dpv);
      if (full) elementwise(st, qb, nb, sv, dpv, cs, cdp, fp, p8[nb], d8[nb], std::false_type{});
      else elementwise(st, qb, nb, sv, dpv, cs, cdp, fp, p8[nb], d8[nb], std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
    // dV^T += dO^T P^T, dK^T += Q^T dS^T over the block's 64 queries
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint4 a0, a1, b0, b1;
      tr_frag(st + 3 * kBlkB, tro.off[db], a0, a1);
      tr_frag(st + kBlkB, tro.off[db], b0, b1);
      dv[db] = mfma8<kFmtE5m2, kFmtE4m3>(a0, a1, p8[0], p8[1], dv[db]);
      dk[db] = mfma8<kFmtE4m3, kFmtE5m2>(b0, b1, d8[0], d8[1], dk[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (n_steps > 0) load_stage(qb0, lds);
  for (int it = 0; it < n_steps; ++it) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    with_slots(lds + ((it + 1) & 1) * kStage, lds + (it & 1) * kStage,
               [&](uint8_t* w, const uint8_t* r) __attribute__((always_inline)) {
                 if (it + 1 < n_steps) load_stage(qb0 + it + 1, w);
                 step(qb0 + it, r);
               });
  }

  if (my_key < Nk) {
    // the lane's half, recomputed from the lane id rather than kept live
    // through the loop
    const int h2 = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5;
    store_rows_bf16((uint16_t*)p.dk + (k_row0 + my_key) * kD, dk, p.scale * sq_max, h2);
    store_rows_bf16((uint16_t*)p.dv + (k_row0 + my_key) * kD, dv, sdo_max / kPScale, h2);
  }
}

// ---------------------------------------------------------------------------
// dQ: a workgroup of 4 waves owns 128 queries (one Q/dO scale tile); 64-key
// blocks of K (rows8 and tr8) and V (rows8) stream through a 2-slot ring.
// Each lane's query is one column of S^T, so its L2 and delta are per-lane
// constants.
// ---------------------------------------------------------------------------
constexpr int kStageQ = 3 * kBlkB;

template <bool CAUSAL>
__device__ __forceinline__ void dq8_body(const Bwd8Params& p, const int head, const int qt) {
  constexpr int DB = kD / 32;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int Nq = p.Nq, Nk = p.Nk;
  const int nqt = (Nq + kScaleRows - 1) / kScaleRows, nkt = (Nk + kScaleRows - 1) / kScaleRows;
  const int q0 = qt * kScaleRows, my_q = q0 + 32 * wv + c;
  const int qw_first = q0 + 32 * wv;  // the wave's first query
  const int64_t q_row0 = (int64_t)head * Nq, k_row0 = (int64_t)head * Nk;
  const float* sk = p.k_scale + (int64_t)head * nkt;
  const float* sv = p.v_scale + (int64_t)head * nkt;
  const float sk_max = scale_max(sk, nkt, lane), rsk = recip_or_zero(sk_max);
  const float sqt = load_uniform(p.q_scale, (int64_t)head * nqt + qt);
  const float sdot = load_uniform(p.do_scale, (int64_t)head * nqt + qt);

  // this wave's Q and dO rows (query my_q) as B operands, and its L2, delta
  uint4 qf[2][2], df[2][2];
  const int qq = min(my_q, Nq - 1);
  {
    const uint8_t* qr = p.q + (q_row0 + qq) * kRowB + 32 * hh;
    const uint8_t* dr = p.do8 + (q_row0 + qq) * kRowB + 32 * hh;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      qf[ks][0] = *(const uint4*)(qr + 64 * ks);
      qf[ks][1] = *(const uint4*)(qr + 64 * ks + 16);
      df[ks][0] = *(const uint4*)(dr + 64 * ks);
      df[ks][1] = *(const uint4*)(dr + 64 * ks + 16);
    }
  }
  const float L = p.stats[q_row0 + qq];
  const float delta = p.stats[(int64_t)p.B * p.H * Nq + q_row0 + qq];
  const bool q_ok = (my_q < Nq) & (L > -INFINITY);
  const TrOffsets tro(lane);
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};

  int n_kb = (Nk + kBlk - 1) / kBlk;
  if (CAUSAL) n_kb = min(n_kb, (min(q0 + kScaleRows, Nq) - 1) / kBlk + 1);
  // waves 0, 1, 2 load K rows8, K tr8, V rows8 of a stage
  const TileLane tlane(lane, wv == 1);
  const uint8_t* tile_src = (wv < 2 ? p.k : p.v) + k_row0 * kRowB;
  auto load_stage = [&](int kb, uint8_t* st) __attribute__((always_inline)) {
    if (wv < 3) load_tile64(tile_src, kb * kBlk, Nk, st + wv * kBlkB, tlane, wv == 1, lane);
  };

  // dS^T of key rows 32 mb .. of block kb, packed four keys (one dword) at a
  // time: element i is key kb*64 + 32 mb + 8 (i/4) + 4 hh + i%4.  MASK: the
  // block is cut by the causal diagonal or an end of the sequences.
  auto half_step = [&](const uint8_t* st, const int kb, const int mb, const float cs, const float cdp,
                       const float dl, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16_t s = f32x16_t{}, dpa = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 a0, a1, b0, b1;
      row_frag(st, mb * 32 + c, ks, hh, a0, a1);
      row_frag(st + 2 * kBlkB, mb * 32 + c, ks, hh, b0, b1);
      s = mfma8<kFmtE4m3, kFmtE4m3>(a0, a1, qf[ks][0], qf[ks][1], s);
      dpa = mfma8<kFmtE4m3, kFmtE5m2>(b0, b1, df[ks][0], df[ks][1], dpa);
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t dw[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float xs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        float t = __builtin_fmaf(s[i], cs, -L);
        if constexpr (MASK) {
          const int key = kb * kBlk + 32 * mb + 8 * g + 4 * hh + j;
          const bool ok = q_ok & (key < Nk) & (!CAUSAL | (key <= my_q));
          t = ok ? t : -INFINITY;
        }
        const float pv = __builtin_amdgcn_exp2f(t);
        xs[j] = clamp_e5m2(pv * __builtin_fmaf(dpa[i], cdp, -dl));
      }
      dw[g] = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(
          xs[2], xs[3], __builtin_amdgcn_cvt_pk_bf8_f32(xs[0], xs[1], __builtin_bit_cast(int, xs[0]), false), true);
    }
    return make_uint4(dw[0], dw[1], dw[2], dw[3]);
  };

  auto step = [&](const int kb, const uint8_t* st) __attribute__((always_inline)) {
    const int ks_ = (kb * kBlk) / kScaleRows;  // the block's K/V scale tile
    const float skb = load_uniform(sk, ks_);
    const float fk = skb * rsk;
    const float cs = p.c * sqt * skb;
    const float cdp = sdot * load_uniform(sv, ks_) * fk;  // dP, times the dQ fold
    const float dl = delta * fk;                          // delta, times the dQ fold
    const bool full = (kb + 1) * kBlk <= Nk && qw_first + 31 < Nq && (!CAUSAL || kb * kBlk + kBlk - 1 <= qw_first);
    uint4 d8[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (full) d8[mb] = half_step(st, kb, mb, cs, cdp, dl, std::false_type{});
      else d8[mb] = half_step(st, kb, mb, cs, cdp, dl, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
    // dQ^T += K^T dS^T over the block's 64 keys
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint4 a0, a1;
      tr_frag(st + kBlkB, tro.off[db], a0, a1);
      acc[db] = mfma8<kFmtE4m3, kFmtE5m2>(a0, a1, d8[0], d8[1], acc[db]);
    }
  };

  if (n_kb > 0) load_stage(0, lds);
  for (int kb = 0; kb < n_kb; ++kb) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    with_slots(lds + ((kb + 1) & 1) * kStageQ, lds + (kb & 1) * kStageQ,
               [&](uint8_t* w, const uint8_t* r) __attribute__((always_inline)) {
                 if (kb + 1 < n_kb) load_stage(kb + 1, w);
                 step(kb, r);
               });
  }
  if (my_q < Nq) store_rows_bf16((uint16_t*)p.dq + (q_row0 + my_q) * kD, acc, p.scale * sk_max, hh);
}

template <bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(kNW * 64, kNW * 64), amdgpu_waves_per_eu(2, 2)))
bwd8_dkdv_kernel(Bwd8Params p) {
  const int w = xcd_remap(blockIdx.x, p.n_work);
  const int nkt = (p.Nk + kScaleRows - 1) / kScaleRows;
  if constexpr (CAUSAL) {
    // key tiles j and nkt-1-j: together the same work as any other pair
    const int half = (nkt + 1) / 2;
    const int head = w / half, j = w - head * half;
    dkdv8_body<CAUSAL>(p, head, j);
    if (nkt - 1 - j != j) {
      __syncthreads();
      dkdv8_body<CAUSAL>(p, head, nkt - 1 - j);
    }
  } else {
    const int head = w / nkt;
    dkdv8_body<CAUSAL>(p, head, w - head * nkt);
  }
}

template <bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(kNW * 64, kNW * 64), amdgpu_waves_per_eu(2, 2)))
bwd8_dq_kernel(Bwd8Params p) {
  const int w = xcd_remap(blockIdx.x, p.n_work);
  const int nqt = (p.Nq + kScaleRows - 1) / kScaleRows;
  if constexpr (CAUSAL) {
    // query tiles nqt-1-j (the heavier) and j
    const int half = (nqt + 1) / 2;
    const int head = w / half, j = w - head * half;
    dq8_body<CAUSAL>(p, head, nqt - 1 - j);
    if (nqt - 1 - j != j) {
      __syncthreads();
      dq8_body<CAUSAL>(p, head, j);
    }
  } else {
    const int head = w / nqt;
    dq8_body<CAUSAL>(p, head, w - head * nqt);
  }
}

template <typename K>
hipError_t set_lds(K kern, int bytes) {
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <bool CAUSAL>
hipError_t launch_bwd8_c(Bwd8Params p, hipStream_t st) {
  const int64_t heads = (int64_t)p.B * p.H;
  const int64_t nqt = (p.Nq + kScaleRows - 1) / kScaleRows, nkt = (p.Nk + kScaleRows - 1) / kScaleRows;
  static bool attr_set = false;  // idempotent; a benign race between threads
  if (!attr_set) {
    hipError_t e = set_lds(bwd8_dkdv_kernel<CAUSAL>, 2 * kStage);
    if (e == hipSuccess) e = set_lds(bwd8_dq_kernel<CAUSAL>, 2 * kStageQ);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (p.Nq > 0) {
    p.n_work = (int)(heads * nqt);
    hipLaunchKernelGGL(bwd8_prep_kernel, dim3(p.n_work), dim3(kPrepThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.Nk > 0) {
    p.n_work = (int)(heads * (CAUSAL ? (nkt + 1) / 2 : nkt));
    hipLaunchKernelGGL(bwd8_dkdv_kernel<CAUSAL>, dim3(p.n_work), dim3(kNW * 64), 2 * kStage, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.Nq > 0) {
    p.n_work = (int)(heads * (CAUSAL ? (nqt + 1) / 2 : nqt));
    hipLaunchKernelGGL(bwd8_dq_kernel<CAUSAL>, dim3(p.n_work), dim3(kNW * 64), 2 * kStageQ, st, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_fp8(bool causal, const Bwd8Params& p, hipStream_t st) {
  return causal ? launch_bwd8_c<true>(p, st) : launch_bwd8_c<false>(p, st);
}

}  // namespace attn
