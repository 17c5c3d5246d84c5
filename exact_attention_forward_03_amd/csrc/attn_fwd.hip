// Exact attention forward for fp16/bf16 on gfx950 (CDNA4).
//
// One workgroup owns a block of 32*NW query rows of one (batch, head) — or
// one (sequence, head) of a variable-length batch — and streams the keys and
// values through LDS in tiles of BC rows, keeping the online-softmax state in
// registers ("Flash Attention 3：让 GPU 跑满的注意力计算", §2.1 tiling, §2.2
// online softmax, §3.1 one independent query block per workgroup; the
// asynchronous producer of "FlashAttention-3", "Three techniques" §1):
//
// * NW waves per workgroup, each owning 32 query rows; two waves run on each
//   SIMD (one 8-wave workgroup or two 4-wave workgroups per CU), so one
//   wave's softmax can overlap the other's MFMAs.  The LDS fragment reads
//   of each MFMA chain are issued a fixed number of MFMAs ahead, and a wave
//   raises its issue priority while it runs an MFMA chain.
// * K and V tiles go from HBM/L2 straight into LDS (buffer_load_dwordx4 with
//   the lds bit through a resource per tile, or global_load_lds_dwordx4 for
//   paged caches: no staging registers, no LDS write instructions, and for
//   dense tensors no vector instructions at all), through a
//   ring of NS buffers: the load of tile j+NS-1 is issued at step j, so a
//   tile has NS-1 steps to arrive.  Rows are stored unpadded with the
//   16-byte chunks of each row XOR-permuted by a function of the row, which
//   keeps the fragment reads free of bank conflicts.
// * S^T = K Q^T on 32x32x16 MFMA puts P in registers already in the
//   B-operand layout of O^T = V^T P^T.  The V^T operand is read from the
//   row-major V tile with the transposing LDS read (ds_read_b64_tr_b16):
//   within a 16-lane group, lane i receives element i & 3 of the 8-byte
//   pieces read by lanes 4j + i / 4, so 4 lanes reading 4 consecutive rows
//   give every lane 4 consecutive keys of one column.
// * Softmax in base 2 with an integer reference maximum.  For each row the
//   kernel keeps Mx = ceil(max of the scores seen so far, times scale log2 e),
//   a reference M <= Mx, p = 2^(S scale log2 e - M) <= 2^(Mx - M),
//   l = sum p (fp32, unrounded) and O = sum p v.  M only moves when some row
//   of the wave would exceed its reference by more than kLazyBits; then
//   every row's M becomes its Mx and O and l are multiplied by
//   2^(M_old - M_new), an exact power of two.  O / l and
//   lse = (M + log2 l) ln 2 equal the page's recurrence (which rescales by
//   e^{m_old - m_new} at every tile) up to rounding: the reference point of
//   the exponentials does not change the sum they define.
// * P enters the second product rounded to fp16/bf16.  While some row of the
//   wave has little weight accumulated (its mass sits on a few keys, so |O|
//   can be as large as |V|), the rounding residual p - round(p) is multiplied
//   in by a second MFMA pass on the same accumulators, which makes the
//   weights exact to ~16 more bits.
// * Causal masking is top-left (key j visible to query i iff j <= i).  Key
//   tiles entirely above a wave's diagonal are skipped by that wave; tiles
//   entirely above the workgroup's diagonal are never loaded.  Only tiles
//   that cross the diagonal or the end of the keys apply an element mask.
// * Workgroup order: the hardware id is remapped so that consecutive work
//   items — the query tiles of one head — run on the same XCD and share its
//   L2 copy of that head's K and V.  Dense causal launches give each
//   workgroup two query tiles, one that sees the most keys (t) and one that
//   sees the fewest (T-1-t), one after the other: every workgroup then does
//   the same work and the launch needs no dynamic balancing (+18 % over one
//   tile per workgroup in heaviest-first order, measured at N = 4096).
//   Dense non-causal launches pair tiles too when the pairs still cover
//   every CU (one round of workgroups instead of two).  With an even number
//   of heads the two tiles of a pair belong to heads h and h + heads/2, so
//   the workgroups running at one time on an XCD share two heads' K/V.
#include <atomic>
#include <mutex>

#include "attn_device.h"
#include "attn_params.h"
#include "attn_sched.h"
#include "attn_tile.h"

namespace attn {
namespace {

using namespace tile;

// Loop options (bit flags).  kOptPin: the LDS fragment reads are pinned
// kPreD MFMAs ahead of their use by scheduling barriers (left alone, the
// compiler keeps only two in flight and the MFMAs wait on LDS latency).
// kOptPrio: a wave raises its issue priority while it runs an MFMA chain, so
// the chain is not starved by the softmax VALU work of the other wave on the
// SIMD.
constexpr int kOptPin = 1, kOptPrio = 2;
// kOptLateLoad: a step issues its tile loads after the S chain instead of
// before it, so the chain starts at once after the barrier.  Measured: +6 %
// at d = 256 (one wave per SIMD), +9 % for variable-length causal launches
// at d = 128 (4-wave workgroups); -10 % for dense d = 128 launches, whose
// loads need the whole step to land; no change for key-chunk launches.
constexpr int kOptLateLoad = 16;
// kOptPersist (variable-length launches): a persistent grid
// (sched::persistent_items).  Used for batches of more than
// sched::kScanSeqs sequences (whose slot numbering leaves up to B + 1
// empty items per head), where it measured -17 % (d = 64, causal), -15 %
// (d = 256, causal) and -6 % (d = 128, non-causal) at 150 sequences of
// 1..500 rows, 32 heads; not for d = 128 causal launches (+0..5 %) nor for a
// few long sequences, where every variant tried (padded or packed counters,
// claims before or after the item, four sub-queues per XCD, a static
// stride) was 1..10 % slower than the dispatcher.  It gains where one
// workgroup fills a CU; where two 4-wave workgroups share one (d = 128
// causal here, the e4m3 kernel) it measured 2..15 % slower.
constexpr int kOptPersist = 64;

__device__ unsigned int g_queues[sched::kQueueSlots][sched::kQueueWords];

// SPLIT: the keys of each head are cut into p.n_split chunks of p.split_len
// rows; a work item is (head, chunk, query tile) and writes the chunk's
// normalised O and its lse in fp32 to p.o_part / p.lse_part, for the merge
// kernel.  Causal masks use absolute key indices (chunk offset + local).
// KV (with SPLIT, non-causal): kKvPaged* read K and V from a paged cache
// through the page table ("Flash Attention 3：让 GPU 跑满的注意力计算", §5.3
// pairs the method with PagedAttention by first copying the pages into a
// contiguous buffer; here each tile's rows are loaded from their page
// directly, no copy).  Sequence b has p.seqlens_k[b] keys; chunk lengths and
// the page size are multiples of BC, so one tile lies within one page and
// needs one table read.  kKvPagedE4m3 / kKvPagedInt8: the cache holds 8-bit
// codes with one fp32 scale per (token, head) in p.k_scale / p.v_scale (the
// INT8 and FP8 KV caches of §4.1.3 of the same post).  Their tiles are
// loaded into registers, converted exactly to the 16-bit type (every e4m3
// and int8 value is representable) and written to the same LDS tiles; the K
// scale multiplies the scores of its key, the V scale the probability of its
// key as it enters the PV product (l sums the unscaled probabilities).
constexpr int kKvDense = 0, kKvPaged = 1, kKvPagedE4m3 = 2, kKvPagedInt8 = 3;

// 16 8-bit codes (one uint4) -> 16 values of the 16-bit type (two uint4), exactly.
template <int KVQ, typename TT>
__device__ __forceinline__ void decode16(TT t, const uint4& w, uint4& lo, uint4& hi) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (KVQ == kKvPagedE4m3) {
      const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], false);
      const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], true);
      out[2 * i] = pack2(t, a[0], a[1]);
      out[2 * i + 1] = pack2(t, b[0], b[1]);
    } else {
      const uint32_t v = ws[i];
      out[2 * i] = pack2(t, (float)(int8_t)(v & 0xff), (float)(int8_t)((v >> 8) & 0xff));
      out[2 * i + 1] = pack2(t, (float)(int8_t)((v >> 16) & 0xff), (float)(int8_t)(v >> 24));
    }
  }
  lo = make_uint4(out[0], out[1], out[2], out[3]);
  hi = make_uint4(out[4], out[5], out[6], out[7]);
}

template <typename TT, int D, int BC, int NW, int WPE, int NS, int OPT, bool CAUSAL, bool VARLEN, bool SPLIT,
          int KV>
__device__ __forceinline__ void attn_fwd_body(const FwdParams& p, const int work) {
  constexpr bool PAGED = KV != kKvDense;
  constexpr int KVQ = KV >= kKvPagedE4m3 ? KV : 0;  // 8-bit cache kind, 0 for 16-bit
  static_assert(!(SPLIT && VARLEN), "key chunks are for dense batches");
  static_assert(!PAGED || (SPLIT && !CAUSAL), "paged caches are read by non-causal key-chunk launches");
  constexpr bool PIN = OPT & kOptPin, PRIO = OPT & kOptPrio, LATE = OPT & kOptLateLoad;
  constexpr int kPreD = 4;  // LDS fragment reads in flight ahead of their MFMA
  constexpr int NQB = 1;
  using C = PipeCfg<D, NQB, BC, NW, NS>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  WorkItem wi;
  if (!decode_work<C::BR, CAUSAL, VARLEN, SPLIT, PAGED>(p, work, wi)) return;
  const int64_t q_row0 = wi.q_row0, k_row0 = wi.k_row0;
  const int q_len = wi.q_len, k_len = wi.k_len, qt = wi.qt, k_off = wi.k_off, head = wi.head, split = wi.split;
  const int q0 = qt * C::BR;
  const uint16_t* __restrict__ Qp = (const uint16_t*)p.q + q_row0 * D;
  const uint8_t* __restrict__ Kb = (const uint8_t*)p.k + k_row0 * D * 2;
  const uint8_t* __restrict__ Vb = (const uint8_t*)p.v + k_row0 * D * 2;

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int qw0 = q0 + wv * C::QW;  // first query row of this wave

  // ---- Q fragments (B operands), one set per 32-row block ----------------
  uint4 qf[NQB][C::KS];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int q = qw0 + nb * 32 + c;
    const bool ok = q < q_len;
    const uint16_t* qrow = Qp + (int64_t)(ok ? q : 0) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[nb][ks] = ok ? *(const uint4*)(qrow + ks * 16) : zero4();
  }

  int n_kt = (k_len + BC - 1) / BC;
  if (CAUSAL) {
    // last key (local index) that some row of the workgroup sees
    const int last = min(q0 + C::BR, q_len) - 1 - k_off;
    n_kt = last < 0 ? 0 : min(n_kt, last / BC + 1);
  }
  int wave_kt = n_kt;
  if (qw0 >= q_len) {
    wave_kt = 0;
  } else if (CAUSAL) {
    const int last = min(qw0 + C::QW - 1, q_len - 1) - k_off;
    wave_kt = last < 0 ? 0 : min(n_kt, last / BC + 1);
  }

  uint8_t* const ldsK = lds;
  uint8_t* const ldsV = lds + NS * C::TILEB;

  // Direct-to-LDS load of one K (or V) tile into buffer `buf`: the wave's
  // i-th instruction fills the 1 KiB block wv * LOADS/NW + i, i.e. rows
  // RPB * block .. + RPB-1; lane l writes chunk l % CHUNKS of row
  // RPB*block + l / CHUNKS and fetches the logical chunk stored there.  Rows
  // past the end of the keys re-read the last key (finite values, masked).
  constexpr int RPB = 1024 / C::ROWB;  // rows per 1 KiB block
  // Paged: tile kt's first row is row `ka0 mod page_size` of page
  // block_table[b][ka0 / page_size] (ka0 = absolute key of the tile's first
  // row; page indices clamped into the cache); the rows of a tile are H
  // cache rows apart.  Returns the index of that (token, head) row.
  auto paged_row = [&](int kt) -> int64_t {
    const int b = head / p.H, h = head - b * p.H;
    const int ka0 = k_off + kt * BC;
    const int j = ka0 / p.page_size;
    const int pg = min(max(load_uniform(p.block_table, (int64_t)b * p.max_pages + j), 0), p.num_pages - 1);
    return ((int64_t)pg * p.page_size + (ka0 - j * p.page_size)) * p.H + h;
  };
  auto dense_load = [&](const uint8_t* base, uint8_t* ring, int kt, int buf, bool is_v) {
    dense_tile_load<C, BC, NW>(base, ring, kt, buf, is_v, k_len, wv, lane);
  };
  auto load_k = [&](int kt, uint8_t* dst) {
    if constexpr (PAGED) {
      const uint8_t* base = (const uint8_t*)p.k + paged_row(kt) * C::ROWB;
#pragma unroll
      for (int i = 0; i < C::LOADS / NW; ++i) {
        const int blk = wv * (C::LOADS / NW) + i;
        const int r = blk * RPB + lane / C::CHUNKS;
        const int rr = min(r, k_len - 1 - kt * BC);
        const uint8_t* src = base + (int64_t)rr * p.H * C::ROWB + k_chunk<C::CHUNKS>(r, lane % C::CHUNKS) * 16;
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(dst + blk * 1024), 16, 0, 0);
      }
    } else {
      dense_load(Kb, dst, kt, 0, false);
    }
  };
  auto load_v = [&](int kt, uint8_t* dst) {
    if constexpr (PAGED) {
      const uint8_t* base = (const uint8_t*)p.v + paged_row(kt) * C::ROWB;
#pragma unroll
      for (int i = 0; i < C::LOADS / NW; ++i) {
        const int blk = wv * (C::LOADS / NW) + i;
        const int r = blk * RPB + lane / C::CHUNKS;
        const int rr = min(r, k_len - 1 - kt * BC);
        const uint8_t* src = base + (int64_t)rr * p.H * C::ROWB + v_chunk<C::CHUNKS>(r, lane % C::CHUNKS) * 16;
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(dst + blk * 1024), 16, 0, 0);
      }
    } else {
      dense_load(Vb, dst, kt, 0, true);
    }
  };

  // 8-bit caches: tile kt's K and V codes go to registers (gload), then are
  // converted and written to the LDS tiles of a ring slot (cvt_store).  A
  // 16-code piece covers 16 values of one row; lane `tid` takes pieces tid,
  // tid + 64 NW, ... of the K tile followed by the V tile, and threads
  // 0 .. 2 BC-1 the K and V scales of the tile's rows.
  constexpr int PIECES = 2 * BC * D / 16;
  constexpr int PPL = KVQ ? PIECES / (NW * 64) : 1;
  static_assert(!KVQ || PIECES % (NW * 64) == 0, "whole pieces per lane");
  static_assert(!KVQ || 2 * BC <= NW * 64, "one scale per thread");
  uint4 raw[PPL];
  float raw_scale = 0.f;
  float* const ldsS = (float*)(lds + 2 * NS * C::TILEB);  // per slot: BC K scales, BC V scales
  auto gload = [&](int kt) {
    const int64_t row0 = paged_row(kt);
    const int last = k_len - 1 - kt * BC;  // last row of the tile that holds a key
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int g = tid + i * NW * 64;
      const bool isv = g >= PIECES / 2;
      const int gg = isv ? g - PIECES / 2 : g;
      const int r = gg / (D / 16), pc = gg % (D / 16);
      const uint8_t* src = (const uint8_t*)(isv ? p.v : p.k) + (row0 + (int64_t)min(r, last) * p.H) * D + pc * 16;
      raw[i] = *(const uint4*)src;
    }
    if (tid < 2 * BC) {
      const int r = tid % BC;
      raw_scale = (tid < BC ? p.k_scale : p.v_scale)[row0 + (int64_t)min(r, last) * p.H];
    }
  };
  auto cvt_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int g = tid + i * NW * 64;
      const bool isv = g >= PIECES / 2;
      const int gg = isv ? g - PIECES / 2 : g;
      const int r = gg / (D / 16), pc = gg % (D / 16);
      uint4 lo, hi;
      decode16<KVQ>(TT{}, raw[i], lo, hi);
      uint8_t* row = (isv ? ldsV : ldsK) + buf * C::TILEB + r * C::ROWB;
      const int c0 = isv ? v_chunk<C::CHUNKS>(r, 2 * pc) : k_chunk<C::CHUNKS>(r, 2 * pc);
      const int c1 = isv ? v_chunk<C::CHUNKS>(r, 2 * pc + 1) : k_chunk<C::CHUNKS>(r, 2 * pc + 1);
      *(uint4*)(row + c0 * 16) = lo;
      *(uint4*)(row + c1 * 16) = hi;
    }
    if (tid < 2 * BC) ldsS[buf * 2 * BC + tid] = raw_scale;
  };
  // scores times the K scale of their key: lane (c, hh) holds keys
  // mb*32 + 8 g + 4 hh + j at s[mb][4 g + j]
  auto scale_by = [&](const float* sc, f32x16_t (&s)[NQB][C::MB]) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 f = *(const float4*)(sc + mb * 32 + 8 * g + 4 * hh);
        s[0][mb][4 * g + 0] *= f.x;
        s[0][mb][4 * g + 1] *= f.y;
        s[0][mb][4 * g + 2] *= f.z;
        s[0][mb][4 * g + 3] *= f.w;
      }
  };

  const float cs = p.c;
  float M[NQB], l[NQB], Mx[NQB];  // reference max, row sum (relative to M), running integer max
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) { M[nb] = -INFINITY; l[nb] = 0.f; Mx[nb] = -INFINITY; }
  f32x16_t oacc[NQB][C::DB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[nb][db] = f32x16_t{};

  // S^T for the key tile in K buffer kbuf; fragments read kPreD MFMAs ahead
  auto compute_s = [&](const uint8_t* kb, f32x16_t (&s)[NQB][C::MB]) {
    constexpr int N = C::MB * C::KS;
    // step i: key block i % MB (alternating accumulators), k-step i / MB
    auto frag = [&](int i) {
      const int r = (i % C::MB) * 32 + c;
      return *(const uint4*)(kb + r * C::ROWB + k_chunk<C::CHUNKS>(r, 2 * (i / C::MB) + hh) * 16);
    };
    uint4 fr[kPreD];
#pragma unroll
    for (int i = 0; i < kPreD; ++i) fr[i] = frag(i);
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) s[0][mb] = f32x16_t{};
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    if (PIN) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint4 a = fr[i % kPreD];
      s[0][i % C::MB] = mfma32(TT{}, a, qf[0][i / C::MB], s[0][i % C::MB]);
      if (i + kPreD < N) fr[i % kPreD] = frag(i + kPreD);
      if (PIN) __builtin_amdgcn_sched_barrier(0);
    }
    if (PRIO) __builtin_amdgcn_s_setprio(0);
  };

  // Masks, row max, M update (with the rare rescale of O and l).
  auto prepare = [&](int kt, f32x16_t (&s)[NQB][C::MB], float (&m_use)[NQB], bool& masked) {
    const int key0 = kt * BC;
    masked = (key0 + BC > k_len) || (CAUSAL && k_off + key0 + BC - 1 > qw0);
    // four independent max chains (short dependency chains)
    float t4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    const int my_q = qw0 + c;
    if (masked) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + mb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          const bool ok = key < k_len && (!CAUSAL || k_off + key <= my_q);
          s[0][mb][i] = ok ? s[0][mb][i] * cs : -INFINITY;
          t4[i & 3] = fmaxf(t4[i & 3], s[0][mb][i]);
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) t4[i & 3] = fmaxf(t4[i & 3], s[0][mb][i]);
    }
    float tmax = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
    if (!masked) tmax *= cs;
    tmax = max_halves(tmax);
    const float m_cand = __builtin_ceilf(tmax);
    Mx[0] = fmaxf(Mx[0], m_cand);
    if (__any(m_cand > M[0] + kLazyBits)) {
      // every row of the wave moves its reference to its running max
      const float m_new = Mx[0];
      const float alpha = (m_new == M[0]) ? 1.f : __builtin_amdgcn_exp2f(M[0] - m_new);
      l[0] *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[0][db][i] *= alpha;
      M[0] = m_new;
    }
    m_use[0] = (M[0] == -INFINITY) ? 0.f : M[0];
  };

  // exponentials, exact row sum and P^T packing of one tile
  auto exps = [&](int slot, f32x16_t (&s)[NQB][C::MB], const float (&m_use)[NQB], bool masked,
                  uint4 (&pf)[NQB][C::MB][2]) {
    float r4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial sums
    if (masked) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[0][mb][i] = __builtin_amdgcn_exp2f(s[0][mb][i] - m_use[0]);
          r4[i & 3] += s[0][mb][i];
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[0][mb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][mb][i], cs, -m_use[0]));
          r4[i & 3] += s[0][mb][i];
        }
    }
    l[0] += (r4[0] + r4[1]) + (r4[2] + r4[3]);
    if constexpr (KVQ) scale_by(ldsS + slot * 2 * BC + BC, s);  // V scales enter with P
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int b = 8 * h2;
        const f32x16_t& v = s[0][mb];
        pf[0][mb][h2] = make_uint4(pack2(TT{}, v[b + 0], v[b + 1]), pack2(TT{}, v[b + 2], v[b + 3]),
                                   pack2(TT{}, v[b + 4], v[b + 5]), pack2(TT{}, v[b + 6], v[b + 7]));
      }
  };

  // O^T += V^T P^T for the tile in V buffer vbuf; the V^T fragment of
  // (db, 16-key step) comes from two transposing reads (keys 4h.. and
  // 8+4h..), read kPreD MFMAs ahead.
  auto pv_pass = [&](const uint8_t* vb, const uint4 (&pp)[NQB][C::MB][2]) {
    const int g = (lane >> 4) & 1, s4 = lane & 15;
    constexpr int N = C::DB * 2 * C::MB;
    // step i: output block i % DB (alternating accumulators), 16-key step i / DB
    auto frag = [&](int i) {
      const int db = i % C::DB, k16 = i / C::DB;
      const int col = db * 32 + 16 * g + 4 * (s4 & 3);  // element column read by this lane
      const int ch = col >> 3, half = (col >> 2) & 1;
      const int r0 = k16 * 16 + 4 * hh + (s4 >> 2);
      const int r1 = r0 + 8;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(vb + r0 * C::ROWB + v_chunk<C::CHUNKS>(r0, ch) * 16 + half * 8));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(vb + r1 * C::ROWB + v_chunk<C::CHUNKS>(r1, ch) * 16 + half * 8));
      const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
      return make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
    };
    constexpr int PV_PRE = kPreD;  // two LDS reads each
    uint4 fr[PV_PRE];
#pragma unroll
    for (int i = 0; i < PV_PRE; ++i) fr[i] = frag(i);
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    if (PIN) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint4 a = fr[i % PV_PRE];
      const int db = i % C::DB, k16 = i / C::DB;
      oacc[0][db] = mfma32(TT{}, a, pp[0][k16 >> 1][k16 & 1], oacc[0][db]);
      if (i + PV_PRE < N) fr[i % PV_PRE] = frag(i + PV_PRE);
      if (PIN) __builtin_amdgcn_sched_barrier(0);
    }
    if (PRIO) __builtin_amdgcn_s_setprio(0);
  };

  // pl <- the rounding residual p - round16(p) of the packed P in pf
  auto residual = [&](f32x16_t (&s)[NQB][C::MB], const uint4 (&pf)[NQB][C::MB][2], uint4 (&pl)[NQB][C::MB][2]) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int b = 8 * h2;
        const f32x16_t& v = s[0][mb];
        const uint4 r = pf[0][mb][h2];
        pl[0][mb][h2] = make_uint4(residual2(TT{}, r.x, v[b + 0], v[b + 1]), residual2(TT{}, r.y, v[b + 2], v[b + 3]),
                                   residual2(TT{}, r.z, v[b + 4], v[b + 5]), residual2(TT{}, r.w, v[b + 6], v[b + 7]));
      }
  };

  // Softmax and second product of tile kt held in s (its K/V ring slot
  // `slot`, V tile at vb).
  auto softmax_pv = [&](int kt, int slot, const uint8_t* vb, f32x16_t (&s)[NQB][C::MB]) {
    float m_use[NQB];
    bool masked = false;
    uint4 pf[NQB][C::MB][2];
    prepare(kt, s, m_use, masked);
    exps(slot, s, m_use, masked, pf);
    // l against the largest p the row can hold, 2^(Mx - M): the weight sits
    // on fewer than kSplitBelowP keys' worth
    const bool split = __any(l[0] < kSplitBelowP * (Mx[0] == M[0] ? 1.f : __builtin_amdgcn_exp2f(Mx[0] - M[0])));
    // the residual is formed before the first product, so the fp32 P dies
    // there and only the two packed copies stay live through the MFMAs
    uint4 pl[NQB][C::MB][2];
    if (split) residual(s, pf, pl);
    pv_pass(vb, pf);
    if (split) pv_pass(vb, pl);
  };

  if constexpr (KVQ) {
    // tile kt+1 is converted into its slot right after the barrier that
    // frees it, while the codes of tile kt+2 are loaded into registers
    if (n_kt > 0) {
      gload(0);
      cvt_store(0);
    }
    if (n_kt > 1) gload(1);
    int slot = 0;
    for (int kt = 0; kt < n_kt; ++kt) {
      __syncthreads();
      const int nxt = (slot + 1 == NS) ? 0 : slot + 1;
      if (kt + 1 < n_kt) {
        cvt_store(nxt);
        if (kt + 2 < n_kt) gload(kt + 2);
      }
      if (kt < wave_kt) {
        f32x16_t s[NQB][C::MB];
        compute_s(ldsK + slot * C::TILEB, s);
        scale_by(ldsS + slot * 2 * BC, s);
        softmax_pv(kt, slot, ldsV + slot * C::TILEB, s);
      }
      slot = nxt;
    }
  }
  // prologue: tiles 0 .. NS-2 in flight (tile j in ring slot j % NS)
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (!KVQ && j < n_kt) {
      load_k(j, ldsK + j * C::TILEB);
      load_v(j, ldsV + j * C::TILEB);
    }
  int slot = 0;  // ring slot of tile kt
  for (int kt = 0; kt < (KVQ ? 0 : n_kt); ++kt) {
    // tile kt must have landed (its loads are the oldest in flight); later
    // tiles may still be on their way
    if (kt + NS - 2 < n_kt) wait_vm<(NS - 2) * C::LPT>();
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // refill the slot tile kt-1 used (every wave is past it now), before
    // or after this step's S chain.  The slot filled and the slot read are
    // different, passed as restrict pointers: the compiler then knows the
    // reads do not depend on the direct-to-LDS loads just issued and does not
    // wait for them (it would otherwise wait for every outstanding load before
    // the first LDS read, leaving the tile no time to arrive).  The explicit
    // vmcnt wait and barrier above order the reads after the loads of earlier
    // steps.
    const int fs = (slot == 0) ? NS - 1 : slot - 1;
    with_disjoint(ldsK + fs * C::TILEB, ldsV + fs * C::TILEB, ldsK + slot * C::TILEB, ldsV + slot * C::TILEB,
                  [&](uint8_t* kw, uint8_t* vw, const uint8_t* kr, const uint8_t* vr) __attribute__((always_inline)) {
      if (!LATE && kt + NS - 1 < n_kt) {
        load_k(kt + NS - 1, kw);
        load_v(kt + NS - 1, vw);
      }
      f32x16_t s[NQB][C::MB];
      if (kt < wave_kt) compute_s(kr, s);
      if (LATE && kt + NS - 1 < n_kt) {
        load_k(kt + NS - 1, kw);
        load_v(kt + NS - 1, vw);
      }
      if (kt < wave_kt) softmax_pv(kt, slot, vr, s);
    });
    slot = (slot + 1 == NS) ? 0 : slot + 1;
  }

  // ---- epilogue -----------------------------------------------------------
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int my_q = qw0 + nb * 32 + c;
    const float l_tot = sum_halves(l[nb]);
    if (my_q < q_len) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const float lse_v = l_tot > 0.f ? (M[nb] + __log2f(l_tot)) * kLn2 : -INFINITY;
      if constexpr (SPLIT) {
        const int64_t prow = (int64_t)split * p.B * p.H * p.Nq + q_row0 + my_q;
        float* orow = p.o_part + prow * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(float4*)(orow + db * 32 + 8 * g + 4 * hh) =
                make_float4(oacc[nb][db][4 * g + 0] * inv, oacc[nb][db][4 * g + 1] * inv,
                            oacc[nb][db][4 * g + 2] * inv, oacc[nb][db][4 * g + 3] * inv);
        if (hh == 0) p.lse_part[prow] = lse_v;
      } else {
        uint16_t* orow = (uint16_t*)p.o + (q_row0 + my_q) * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dcol = db * 32 + 8 * g + 4 * hh;
            *(uint2*)(orow + dcol) =
                make_uint2(pack2(TT{}, oacc[nb][db][4 * g + 0] * inv, oacc[nb][db][4 * g + 1] * inv),
                           pack2(TT{}, oacc[nb][db][4 * g + 2] * inv, oacc[nb][db][4 * g + 3] * inv));
          }
        if (hh == 0) p.lse[q_row0 + my_q] = lse_v;
      }
    }
  }
}

// The kernel: one work item, or (dense launches with p.pair_tiles) a pair of
// query tiles one after the other (run_items), or (kOptPersist) the items it
// takes from its XCD's queue.
template <typename TT, int D, int BC, int NW, int WPE, int NS, int OPT, bool CAUSAL, bool VARLEN, bool SPLIT,
          int KV>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(WPE, WPE)))
attn_fwd_dma_kernel(FwdParams p) {
  if constexpr (VARLEN && (OPT & kOptPersist)) {
    sched::persistent_items(g_queues[p.queue], p.n_work, [&](int item) __attribute__((always_inline)) {
      attn_fwd_body<TT, D, BC, NW, WPE, NS, OPT, CAUSAL, VARLEN, SPLIT, KV>(p, item);
    });
  } else {
    const int w = xcd_remap(blockIdx.x, p.n_work);
    constexpr bool kPairs = !VARLEN && !SPLIT && KV == kKvDense;
    run_items<kPairs, CAUSAL>(p, w, [&](int item) __attribute__((always_inline)) {
      attn_fwd_body<TT, D, BC, NW, WPE, NS, OPT, CAUSAL, VARLEN, SPLIT, KV>(p, item);
    });
  }
}

template <typename TT, int D, int BC, int NW, int WPE, int NS, int OPT, bool CAUSAL, bool VARLEN, bool SPLIT,
          int KV>
hipError_t launch_dma_one(const FwdParams& p, hipStream_t st) {
  using C = PipeCfg<D, 1, BC, NW, NS>;
  auto kern = attn_fwd_dma_kernel<TT, D, BC, NW, WPE, NS, OPT, CAUSAL, VARLEN, SPLIT, KV>;
  // 8-bit caches add the per-slot row scales after the K and V rings
  constexpr int lds_bytes = C::LDS_BYTES + (KV >= kKvPagedE4m3 ? NS * 2 * BC * 4 : 0);
  static bool attr_set = false;  // idempotent; a benign race between threads
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  FwdParams pp = p;
  if constexpr (!VARLEN && !SPLIT && KV == kKvDense) {
    const hipError_t e = plan_pairs(pp, CAUSAL);
    if (e != hipSuccess) return e;
  } else {
    pp.pair_tiles = 0;
  }
  if (pp.n_work == 0) return hipSuccess;
  unsigned grid = (unsigned)pp.n_work;
  if constexpr (VARLEN && (OPT & kOptPersist)) {
    static std::atomic<int> per_cu{0};
    const hipError_t e = sched::persistent_grid((const void*)kern, NW * 64, lds_bytes, pp.n_work, per_cu, &grid);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), lds_bytes, st, pp);
  return hipGetLastError();
}

// Tile configuration per head dimension and masking: key rows per tile,
// waves per workgroup (query rows = 32 x waves), waves per SIMD, LDS ring
// depth and loop options.  Dense causal launches at d = 128 use the
// non-causal configuration: every workgroup runs a pair of query tiles of
// equal total work (+8 % over 4-wave workgroups with 64-key tiles, measured
// at N = 4096 and 8192).  Variable-length causal launches have no pairs and
// run 4-wave workgroups, two per CU, so that one workgroup's diagonal tiles
// and early exits do not hold a whole 8-wave workgroup at its barriers.
template <int D, bool CAUSAL> struct DmaTile;
template <bool CAUSAL> struct DmaTile<64, CAUSAL> {
  static constexpr int BC = 64, NW = 8, WPE = 2, NS = 3, OPT = kOptPin | kOptPrio;
};
template <bool CAUSAL> struct DmaTile<128, CAUSAL> {
  static constexpr int BC = 128, NW = 8, WPE = 2, NS = 2, OPT = kOptPin | kOptPrio;
};
template <bool CAUSAL> struct DmaTile<256, CAUSAL> {
  static constexpr int BC = 64, NW = 4, WPE = 1, NS = 2, OPT = kOptPin | kOptLateLoad;
};
struct VarlenCausalTile128 {
  static constexpr int BC = 64, NW = 4, WPE = 2, NS = 2, OPT = kOptPin | kOptPrio | kOptLateLoad;
};

// Key-chunk launches at d = 128 (decoding and long keys with few queries):
// 4-wave workgroups with a 64 KiB ring, so two run on each CU.
struct SplitTile128 { static constexpr int BC = 64, NW = 4, WPE = 2, NS = 2, OPT = kOptPin | kOptPrio; };

template <typename TT, int D, bool CAUSAL, bool VARLEN, bool SPLIT, int KV = kKvDense>
hipError_t launch_dma_d(const FwdParams& p, hipStream_t st) {
  using T = DmaTile<D, CAUSAL>;
  if constexpr (SPLIT && D == 128) {
    using S = SplitTile128;
    return launch_dma_one<TT, D, S::BC, S::NW, S::WPE, S::NS, S::OPT, CAUSAL, VARLEN, SPLIT, KV>(p, st);
  } else if constexpr (CAUSAL && VARLEN && D == 128) {
    using V = VarlenCausalTile128;
    return launch_dma_one<TT, D, V::BC, V::NW, V::WPE, V::NS, V::OPT, CAUSAL, VARLEN, SPLIT, KV>(p, st);
  } else if constexpr (VARLEN && !SPLIT) {
    int slot = 0;
    if (p.B > sched::kScanSeqs && sched::queue_slot(st, &slot)) {
      FwdParams pp = p;
      pp.queue = slot;
      return launch_dma_one<TT, D, T::BC, T::NW, T::WPE, T::NS, T::OPT | kOptPersist, CAUSAL, VARLEN, SPLIT, KV>(pp,
                                                                                                              st);
    }
    return launch_dma_one<TT, D, T::BC, T::NW, T::WPE, T::NS, T::OPT, CAUSAL, VARLEN, SPLIT, KV>(p, st);
  } else {
    return launch_dma_one<TT, D, T::BC, T::NW, T::WPE, T::NS, T::OPT, CAUSAL, VARLEN, SPLIT, KV>(p, st);
  }
}

template <typename TT, bool CAUSAL, bool VARLEN, bool SPLIT, int KV = kKvDense>
hipError_t launch_dma_cv(int d, const FwdParams& p, hipStream_t st) {
  switch (d) {
    case 64: return launch_dma_d<TT, 64, CAUSAL, VARLEN, SPLIT, KV>(p, st);
    case 128: return launch_dma_d<TT, 128, CAUSAL, VARLEN, SPLIT, KV>(p, st);
    case 256: return launch_dma_d<TT, 256, CAUSAL, VARLEN, SPLIT, KV>(p, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename TT>
hipError_t launch_dma_t(int d, bool causal, bool varlen, bool split, int kv, const FwdParams& p,
                        hipStream_t st) {
  if (kv != kKvDense) {
    if (!split || varlen || causal) return hipErrorInvalidValue;
    switch (kv) {
      case kKvPaged: return launch_dma_cv<TT, false, false, true, kKvPaged>(d, p, st);
      case kKvPagedE4m3: return launch_dma_cv<TT, false, false, true, kKvPagedE4m3>(d, p, st);
      case kKvPagedInt8: return launch_dma_cv<TT, false, false, true, kKvPagedInt8>(d, p, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (split) {
    if (varlen) return hipErrorInvalidValue;
    return causal ? launch_dma_cv<TT, true, false, true>(d, p, st) : launch_dma_cv<TT, false, false, true>(d, p, st);
  }
  if (causal)
    return varlen ? launch_dma_cv<TT, true, true, false>(d, p, st) : launch_dma_cv<TT, true, false, false>(d, p, st);
  return varlen ? launch_dma_cv<TT, false, true, false>(d, p, st) : launch_dma_cv<TT, false, false, false>(d, p, st);
}

}  // namespace

// One slot per stream: launches on one stream run one after the other, so
// any two launches that may run together have different slots (a stream
// destroyed while its launch still runs and a new stream given the same
// handle are the exception).
bool sched::queue_slot(hipStream_t st, int* slot) {
  if (st == hipStreamPerThread) return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();  // the launch reports its own errors
    return false;
  }
  if (cs != hipStreamCaptureStatusNone) return false;
  static std::mutex mu;
  static hipStream_t owner[kQueueSlots];
  static int used = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (owner[i] == st) {
      *slot = i;
      return true;
    }
  if (used == kQueueSlots) return false;
  owner[used] = st;
  *slot = used++;
  return true;
}

// Compute units of the current device, asked of the runtime once per device
// (the launch decides on it for every dense non-causal call).
hipError_t tile::device_cu_count(int* cus) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0: not asked yet
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) cache[dev].store(*cus, std::memory_order_relaxed);
  return e;
}

int fwd_split_block_rows(int dtype, int d, bool causal) {
  if (d == 128) return 32 * SplitTile128::NW;
  return fwd_block_rows(dtype, d, causal, false);
}

int fwd_block_rows(int dtype, int d, bool causal, bool varlen) {
  if (dtype == 2) return fwd_fp8_block_rows(causal);
  switch (d) {
    case 64: return 32 * DmaTile<64, false>::NW;
    case 128:
      if (causal && varlen) return 32 * VarlenCausalTile128::NW;
      return causal ? 32 * DmaTile<128, true>::NW : 32 * DmaTile<128, false>::NW;
    default: return 32 * DmaTile<256, false>::NW;
  }
}

int fwd_split_tile_keys(int d) {
  switch (d) {
    case 64: return DmaTile<64, false>::BC;
    case 128: return SplitTile128::BC;
    default: return DmaTile<256, false>::BC;
  }
}

hipError_t launch_fwd(int dtype, int d, bool causal, bool varlen, bool split, int kv, const FwdParams& p,
                      hipStream_t st) {
  if (split && decode_shape(p.Nq, kv)) return launch_decode(dtype, d, causal, kv, p, st);
  if (dtype == 0) return launch_dma_t<f16_t>(d, causal, varlen, split, kv, p, st);
  return launch_dma_t<bf16_t>(d, causal, varlen, split, kv, p, st);
}

}  // namespace attn
