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
// clamped to +-57344 first).
__device__ __forceinline__ uint4 pack16_e4m3(const f32x16_t& v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i], v[4 * i + 1], 0, false);
    w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i + 2], v[4 * i + 3], x, true);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ float clamp_e5m2(float x) { return fminf(fmaxf(x, -kE5m2Max), kE5m2Max); }
__device__ __forceinline__ uint4 pack16_e5m2(const f32x16_t& v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int x = __builtin_amdgcn_cvt_pk_bf8_f32(clamp_e5m2(v[4 * i]), clamp_e5m2(v[4 * i + 1]), 0, false);
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
  return m;
}

// Direct-to-LDS load of 1 KiB block b (8 rows) of a 64-row tile: rows
// r0 + 8 b .. of src (codes, rows of 128 bytes; rows past n_rows re-read
// the last row), chunk-permuted by perm.
template <bool TR>
__device__ __forceinline__ void load_block8(const uint8_t* src, int64_t row_base, int r0, int n_rows, uint8_t* dst,
                                            int b, int lane) {
  const int r = 8 * b + (lane >> 3);
  const int row = min(r0 + r, n_rows - 1);
  const int ch = TR ? tr8(r, lane & 7) : rows8(r, lane & 7);
  __builtin_amdgcn_global_load_lds(src + (row_base + row) * kRowB + ch * 16, (lds_void_t*)(dst + b * 1024), 16, 0,
                                   0);
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
// delta_i = sum_c dO_ic O_ic in fp32; s = amax(dO tile) / 57344 (1 if the
// tile is all zero, at least 2^-149); codes e5m2(dO / s).  Two threads per
// row, 64 values each.
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 256;

__global__ void __launch_bounds__(kPrepThreads) bwd8_prep_kernel(Bwd8Params p) {
  __shared__ float red[kPrepThreads / 64];
  const int nt = (p.Nq + kScaleRows - 1) / kScaleRows;
  const int bh = blockIdx.x / nt, tile = blockIdx.x - bh * nt;
  const int row = tile * kScaleRows + (threadIdx.x >> 1), half = threadIdx.x & 1;
  const bool live = row < p.Nq;
  const int64_t base = ((int64_t)bh * p.Nq + (live ? row : 0)) * kD + half * 64;
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
  if (live && half == 0) p.delta[(int64_t)bh * p.Nq + row] = dsum;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s));
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
// head; 64-row blocks of Q and dO (each stored twice: rows8 and tr8), lse
// and delta stream through a 2-slot LDS ring.
// ---------------------------------------------------------------------------
constexpr int kNW = 4;
constexpr int kStage = 4 * kBlkB + 2 * kBlk * 4;  // Q rows8, Q tr8, dO rows8, dO tr8, lse[64], delta[64]

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
  const int64_t q_row0 = (int64_t)head * Nq, k_row0 = (int64_t)head * Nk;
  const float* sq = p.q_scale + (int64_t)head * nqt;
  const float* sdo = p.do_scale + (int64_t)head * nqt;
  const float sq_max = scale_max(sq, nqt, lane), sdo_max = scale_max(sdo, nqt, lane);
  const float skt = p.k_scale[(int64_t)head * nkt + kt], svt = p.v_scale[(int64_t)head * nkt + kt];

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
  auto load_stage = [&](int qb, uint8_t* st) {
    // 32 blocks of 1 KiB (four 8 KiB tiles), eight per wave
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int blk = wv * 8 + i, tile = blk >> 3, b = blk & 7;
      const uint8_t* src = tile < 2 ? p.q : p.do8;
      if (tile & 1) load_block8<true>(src, q_row0, qb * kBlk, Nq, st + tile * kBlkB, b, lane);
      else load_block8<false>(src, q_row0, qb * kBlk, Nq, st + tile * kBlkB, b, lane);
    }
    if (wv < 2) {  // lse (wave 0) and delta (wave 1): 64 floats each, 4-byte loads
      const int q = min(qb * kBlk + lane, Nq - 1);
      const float* src = (wv == 0 ? p.lse : p.delta) + q_row0 + q;
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(st + 4 * kBlkB + wv * 256), 4, 0, 0);
    }
  };

  if (n_steps > 0) load_stage(qb0, lds);
  for (int it = 0; it < n_steps; ++it) {
    const int qb = qb0 + it;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint8_t* const st = lds + (it & 1) * kStage;
    if (it + 1 < n_steps) load_stage(qb + 1, lds + ((it + 1) & 1) * kStage);
    const uint8_t* tq = st;
    const uint8_t* tqT = st + kBlkB;
    const uint8_t* tdo = st + 2 * kBlkB;
    const uint8_t* tdoT = st + 3 * kBlkB;
    const float* tl = (const float*)(st + 4 * kBlkB);
    const float* tdl = tl + kBlk;

    const int qs = (qb * kBlk) / kScaleRows;  // the block's scale tile
    const float sqb = load_uniform(sq, qs), sdob = load_uniform(sdo, qs);
    const float cs = p.c * sqb * skt;  // S in base 2
    const float cdp = sdob * svt;
    const float fp = kPScale * (sdob / sdo_max);
    const float fs = sqb / sq_max;

    // S = Q K^T and dP = dO V^T for query rows 32 nb .. of the block
    f32x16_t s[2], dpa[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      s[nb] = f32x16_t{};
      dpa[nb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 a0, a1;
        row_frag(tq, nb * 32 + c, ks, hh, a0, a1);
        s[nb] = mfma8<kFmtE4m3, kFmtE4m3>(a0, a1, kf[ks][0], kf[ks][1], s[nb]);
        row_frag(tdo, nb * 32 + c, ks, hh, a0, a1);
        dpa[nb] = mfma8<kFmtE5m2, kFmtE4m3>(a0, a1, vf[ks][0], vf[ks][1], dpa[nb]);
      }
    }
    // P, dS; element (nb, i) is query qb*64 + 32 nb + 8 (i/4) + 4 hh + i%4
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * nb + 8 * (i >> 2) + 4 * hh + (i & 3);
        const int q = qb * kBlk + r;
        const float L = tl[r];
        const bool ok = q < Nq && my_key < Nk && (!CAUSAL || my_key <= q) && L > -INFINITY;
        const float pv = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][i], cs, -L * kLog2e)) : 0.f;
        const float ds = pv * __builtin_fmaf(dpa[nb][i], cdp, -tdl[r]);
        s[nb][i] = pv * fp;
        dpa[nb][i] = ds * fs;
      }
    }
    const uint4 p0 = pack16_e4m3(s[0]), p1 = pack16_e4m3(s[1]);
    const uint4 d0 = pack16_e5m2(dpa[0]), d1 = pack16_e5m2(dpa[1]);
    // dV^T += dO^T P^T, dK^T += Q^T dS^T over the block's 64 queries
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint4 a0, a1;
      tr_frag(tdoT, tro.off[db], a0, a1);
      dv[db] = mfma8<kFmtE5m2, kFmtE4m3>(a0, a1, p0, p1, dv[db]);
      tr_frag(tqT, tro.off[db], a0, a1);
      dk[db] = mfma8<kFmtE4m3, kFmtE5m2>(a0, a1, d0, d1, dk[db]);
    }
  }

  if (my_key < Nk) {
    store_rows_bf16((uint16_t*)p.dk + (k_row0 + my_key) * kD, dk, p.scale * sq_max, hh);
    store_rows_bf16((uint16_t*)p.dv + (k_row0 + my_key) * kD, dv, sdo_max / kPScale, hh);
  }
}

// ---------------------------------------------------------------------------
// dQ: a workgroup of 4 waves owns 128 queries (one Q/dO scale tile); 64-key
// blocks of K (rows8 and tr8) and V (rows8) stream through a 2-slot ring.
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
  const int64_t q_row0 = (int64_t)head * Nq, k_row0 = (int64_t)head * Nk;
  const float* sk = p.k_scale + (int64_t)head * nkt;
  const float* sv = p.v_scale + (int64_t)head * nkt;
  const float sk_max = scale_max(sk, nkt, lane);
  const float sqt = p.q_scale[(int64_t)head * nqt + qt], sdot = p.do_scale[(int64_t)head * nqt + qt];

  // this wave's Q and dO rows (query my_q) as B operands, and its lse, delta
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
  const float L = p.lse[q_row0 + qq], dl = p.delta[q_row0 + qq];
  const bool q_ok = my_q < Nq && L > -INFINITY;
  const TrOffsets tro(lane);
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};

  int n_kb = (Nk + kBlk - 1) / kBlk;
  if (CAUSAL) n_kb = min(n_kb, (min(q0 + kScaleRows, Nq) - 1) / kBlk + 1);
  auto load_stage = [&](int kb, uint8_t* st) {
    // 24 blocks of 1 KiB (K rows8, K tr8, V rows8), six per wave
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int blk = wv * 6 + i, tile = blk >> 3, b = blk & 7;
      const uint8_t* src = tile < 2 ? p.k : p.v;
      if (tile == 1) load_block8<true>(src, k_row0, kb * kBlk, Nk, st + tile * kBlkB, b, lane);
      else load_block8<false>(src, k_row0, kb * kBlk, Nk, st + tile * kBlkB, b, lane);
    }
  };

  if (n_kb > 0) load_stage(0, lds);
  for (int kb = 0; kb < n_kb; ++kb) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint8_t* const st = lds + (kb & 1) * kStageQ;
    if (kb + 1 < n_kb) load_stage(kb + 1, lds + ((kb + 1) & 1) * kStageQ);
    const uint8_t* tk = st;
    const uint8_t* tkT = st + kBlkB;
    const uint8_t* tv = st + 2 * kBlkB;

    const int ks_ = (kb * kBlk) / kScaleRows;  // the block's K/V scale tile
    const float skb = load_uniform(sk, ks_);
    const float cs = p.c * sqt * skb;
    const float cdp = sdot * load_uniform(sv, ks_);
    const float fk = skb / sk_max;
    // S^T = K Q^T and dP^T = V dO^T for key rows 32 mb .. of the block
    f32x16_t s[2], dpa[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16_t{};
      dpa[mb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 a0, a1;
        row_frag(tk, mb * 32 + c, ks, hh, a0, a1);
        s[mb] = mfma8<kFmtE4m3, kFmtE4m3>(a0, a1, qf[ks][0], qf[ks][1], s[mb]);
        row_frag(tv, mb * 32 + c, ks, hh, a0, a1);
        dpa[mb] = mfma8<kFmtE4m3, kFmtE5m2>(a0, a1, df[ks][0], df[ks][1], dpa[mb]);
      }
    }
    // element (mb, i) is key kb*64 + 32 mb + 8 (i/4) + 4 hh + i%4
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * kBlk + 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
        const bool ok = q_ok && key < Nk && (!CAUSAL || key <= my_q);
        const float pv = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][i], cs, -L * kLog2e)) : 0.f;
        dpa[mb][i] = pv * __builtin_fmaf(dpa[mb][i], cdp, -dl) * fk;
      }
    }
    const uint4 d0 = pack16_e5m2(dpa[0]), d1 = pack16_e5m2(dpa[1]);
    // dQ^T += K^T dS^T over the block's 64 keys
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint4 a0, a1;
      tr_frag(tkT, tro.off[db], a0, a1);
      acc[db] = mfma8<kFmtE4m3, kFmtE5m2>(a0, a1, d0, d1, acc[db]);
    }
  }
  if (my_q < Nq) store_rows_bf16((uint16_t*)p.dq + (q_row0 + my_q) * kD, acc, p.scale * sk_max, hh);
}

template <bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(kNW * 64, kNW * 64))) bwd8_dkdv_kernel(Bwd8Params p) {
  const int w = xcd_remap(blockIdx.x, p.n_work);
  const int nkt = (p.Nk + kScaleRows - 1) / kScaleRows;
  const int head = w / nkt;
  dkdv8_body<CAUSAL>(p, head, w - head * nkt);
}

template <bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(kNW * 64, kNW * 64))) bwd8_dq_kernel(Bwd8Params p) {
  const int w = xcd_remap(blockIdx.x, p.n_work);
  const int nqt = (p.Nq + kScaleRows - 1) / kScaleRows;
  const int head = w / nqt;
  dq8_body<CAUSAL>(p, head, w - head * nqt);
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
    p.n_work = (int)(heads * nkt);
    hipLaunchKernelGGL(bwd8_dkdv_kernel<CAUSAL>, dim3(p.n_work), dim3(kNW * 64), 2 * kStage, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.Nq > 0) {
    p.n_work = (int)(heads * nqt);
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
