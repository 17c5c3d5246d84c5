// Tile geometry, LDS layouts, work decomposition and tile loads shared by
// the fp16/bf16 forward kernels (attn_fwd.hip): one workgroup streams the K
// and V tiles of one (batch, head) or (sequence, head) through a ring of LDS
// buffers ("Flash Attention 3：让 GPU 跑满的注意力计算", §2.1 tiling, §3.1 one
// independent query block per workgroup).
#pragma once

#include "attn_device.h"
#include "attn_params.h"
#include "attn_sched.h"

namespace attn {
namespace tile {

// The rounding residual of P is multiplied in while some row of a wave has
// accumulated less weight than kSplitBelowP times its largest possible p.
constexpr float kSplitBelowP = 8.0f;
// Slack of the reference max M: a row's scores may exceed M by up to
// kLazyBits (p = 2^(t - M) <= 2^kLazyBits) before the wave rescales O and l.
// O and lse do not depend on M (up to rounding); on N(0,1) scores this takes
// a wave's rescales from about every second key tile to almost none.
constexpr float kLazyBits = 4.0f;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int D, int NQB, int BC, int NW, int NS>
struct PipeCfg {
  static constexpr int QW = NQB * 32;        // query rows per wave
  static constexpr int BR = NW * QW;         // query rows per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int ROWB = D * 2;         // bytes per K/V row in LDS (unpadded)
  static constexpr int CHUNKS = ROWB / 16;   // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;    // bytes per K or V tile
  static constexpr int KS = D / 16;          // MFMA k-steps of S^T
  static constexpr int MB = BC / 32;         // 32-key blocks per tile
  static constexpr int DB = D / 32;          // 32-row blocks of O^T
  static constexpr int LOADS = TILEB / 1024; // 1 KiB direct-to-LDS loads per tile
  static constexpr int LDS_BYTES = 2 * NS * TILEB;  // K and V rings of NS slots
  static constexpr int LPT = 2 * LOADS / NW;  // load instructions per wave per tile (K and V)
  static_assert(LOADS % NW == 0, "each wave issues the same number of tile loads");
  static_assert(CHUNKS >= 8, "row swizzle needs at least 8 chunks");
};

// Physical 16-byte chunk of logical chunk `ch` in K row `r`: all 16 rows of
// an aligned group land on different chunks (K fragment reads: 16 lanes,
// 16 rows, same logical chunk).
template <int CHUNKS>
__device__ __forceinline__ int k_chunk(int r, int ch) { return ch ^ (r & (CHUNKS >= 16 ? 15 : 7)); }
// V rows: a transposing read of 32 lanes covers 4 consecutive rows x 4
// neighbouring chunks (two 16-lane groups, 2 chunks each); XOR-ing with
// (row & 3) << 2 puts them on 16 different chunks.  Rows of 8 chunks (d = 64)
// use (row & 3) << 1.
template <int CHUNKS>
__device__ __forceinline__ int v_chunk(int r, int ch) { return ch ^ ((r & 3) << (CHUNKS >= 16 ? 2 : 1)); }


// One work item of a launch: a block of query rows of one (batch, head), of
// one (sequence, head) of a variable-length batch, or of one (head, key
// chunk), and the key range it sees.
struct WorkItem {
  int64_t q_row0, k_row0;  // row of the head's (sequence's) first query in Q/O and first key in K/V
  int q_len, k_len;        // queries and keys of that head (sequence, key chunk)
  int qt;                  // query tile (heaviest first for causal launches)
  int k_off;               // absolute index of the range's first key (key chunks), else 0
  int head, split;         // flat (batch, head) or head index; key chunk
};

// work index -> item; false for the surplus items of variable-length
// launches (their grid is an upper bound).  BR: query rows per item.
// work = head * tiles_per_head + t: t is a query tile (dense), or a slot of
// the head's query tiles (variable-length batches, sched::slot_tile).
template <int BR, bool CAUSAL, bool VARLEN, bool SPLIT, bool PAGED>
__device__ __forceinline__ bool decode_work(const FwdParams& p, const int work, WorkItem& w) {
  const int hs = work / p.tiles_per_head;  // head, or head * n_split + chunk
  const int t = work - hs * p.tiles_per_head;
  const int head = SPLIT ? hs / p.n_split : hs;
  const int split = SPLIT ? hs - head * p.n_split : 0;
  w.head = head;
  w.split = split;
  w.k_off = 0;
  if constexpr (!VARLEN) {
    w.q_len = p.Nq;
    w.q_row0 = (int64_t)head * p.Nq;
    if constexpr (SPLIT) {
      int64_t nk = p.Nk;
      if constexpr (PAGED)
        nk = min(max(load_uniform(p.seqlens_k, head / p.H), 0), p.max_pages * p.page_size);
      const int64_t kb = min((int64_t)split * p.split_len, nk);
      const int64_t ke = min(kb + p.split_len, nk);
      w.k_off = (int)kb;
      w.k_len = (int)(ke - kb);
    } else {
      w.k_len = p.Nk;
    }
    w.k_row0 = PAGED ? 0 : (int64_t)head * p.Nk + w.k_off;
    w.qt = CAUSAL ? (p.tiles_per_head - 1 - t) : t;
  } else {
    sched::SlotTile st;
    if (!sched::find_tile<BR>(p.cu_q, p.B, p.Nq, p.cu_k, p.Nk, t, st)) return false;
    const int nts = (st.e - st.a + BR - 1) / BR;
    w.qt = CAUSAL ? (nts - 1 - st.j) : st.j;  // causal: a sequence's heaviest tile first
    w.q_len = st.e - st.a;
    w.k_len = st.oe - st.oa;
    w.q_row0 = (int64_t)head * p.Nq + st.a;
    w.k_row0 = (int64_t)head * p.Nk + st.oa;
  }
  return true;
}

// Dense K or V tile kt -> ring buffer `buf`: the wave's i-th load fills
// 1 KiB block i * NW + wv.  The rows come through a buffer resource based at
// the tile's first key, so the per-lane byte offset (row within the block,
// swizzled chunk) is the same for every tile and the block offset is a
// wave-uniform scalar: a full tile costs no vector instructions.  The
// resource covers only the tile's keys; the last tile, when it runs past
// them, clamps its rows per lane to the last key, so no read goes out of
// range.
template <typename C, int BC, int NW>
__device__ __forceinline__ void dense_tile_load(const uint8_t* base, uint8_t* ring, int kt, int buf, bool is_v,
                                                int k_len, int wv, int lane) {
  constexpr int RPB = 1024 / C::ROWB;  // rows per 1 KiB block
  auto chunk = [&](int r, int ch) { return is_v ? v_chunk<C::CHUNKS>(r, ch) : k_chunk<C::CHUNKS>(r, ch); };
  const int rows = min(BC, k_len - kt * BC);  // >= 1: only tiles holding keys are loaded
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + (int64_t)kt * BC * C::ROWB), 0, rows * C::ROWB, kBufferFlags);
  if (rows == BC) {
#pragma unroll
    for (int i = 0; i < C::LOADS / NW; ++i) {
      const int blk = i * NW + wv;
      // the swizzles read the row mod 16, which is the same for every i
      // when a round of NW blocks spans a multiple of 16 rows
      const int r = (NW * RPB) % 16 == 0 ? wv * RPB + lane / C::CHUNKS : blk * RPB + lane / C::CHUNKS;
      const uint32_t voff = (uint32_t)((lane / C::CHUNKS) * C::ROWB + chunk(r, lane % C::CHUNKS) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(ring + buf * C::TILEB + blk * 1024), 16, voff,
                                               (uint32_t)(blk * 1024), 0, 0);
    }
  } else {
    // the lane index through an empty asm: the per-lane rows and chunks of
    // this rare path are then computed here, not hoisted out of the tile
    // loop to occupy registers (or scratch) for the whole kernel
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < C::LOADS / NW; ++i) {
      const int blk = i * NW + wv;
      const int r = blk * RPB + ln / C::CHUNKS;
      const uint32_t voff = (uint32_t)(min(r, rows - 1) * C::ROWB + chunk(r, ln % C::CHUNKS) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(ring + buf * C::TILEB + blk * 1024), 16, voff,
                                               0, 0, 0);
    }
  }
}


// Runs the work of workgroup w.  One work item, or, for dense launches with
// p.pair_tiles, two query tiles one after the other (p.n_work counts pairs
// then).  With an even number of heads the pair is tile t of head h and the
// partner tile of head h + heads/2, so the workgroups running at one time on
// an XCD share two heads' K/V in its L2 (as unpaired launches do), not four;
// otherwise it is tiles t and T-1-t of one head (with an odd tile count the
// middle tile runs alone).  The partner of a causal tile t is T-1-t (qt =
// T-1-t in the heaviest-first numbering is tile t, and the other way round),
// so every workgroup does the same work; causal launches always pair.
// Non-causal launches pair when the pairs still cover every CU: one round of
// workgroups instead of two, which takes the tail of the second round off
// (N=4096, d=128: 316 -> 305 us).
template <bool PAIRS, bool CAUSAL, typename Run>
__device__ __forceinline__ void run_items(const FwdParams& p, const int w, Run&& run) {
  if constexpr (PAIRS) {
    if (CAUSAL || p.pair_tiles) {
      const int T = p.tiles_per_head, heads = p.B * p.H;
      if (heads % 2 == 0) {
        const int h = w / T, t = w - h * T;
        run(h * T + t);
        __syncthreads();
        run((h + heads / 2) * T + (CAUSAL ? T - 1 - t : t));
      } else {
        const int half = (T + 1) / 2;
        const int head = w / half, t = w - head * half;
        run(head * T + t);
        if (T - 1 - t != t) {
          __syncthreads();
          run(head * T + (T - 1 - t));
        }
      }
      return;
    }
  }
  run(w);
}

// Compute units of the current device, asked of the runtime once per device.
hipError_t device_cu_count(int* cus);

// Host: decides whether a dense launch runs pairs of query tiles (run_items)
// and sets pp.pair_tiles and pp.n_work (workgroups) accordingly.
inline hipError_t plan_pairs(FwdParams& pp, bool causal) {
  pp.pair_tiles = 0;
  const int64_t heads = pp.n_work / pp.tiles_per_head;
  const int64_t pairs =
      heads % 2 == 0 ? heads / 2 * pp.tiles_per_head : heads * ((pp.tiles_per_head + 1) / 2);
  bool pair = causal;
  if (!causal) {
    int cus = 0;
    const hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    pair = pairs >= cus;
  }
  if (pair) {
    pp.pair_tiles = 1;
    pp.n_work = (int)pairs;
  }
  return hipSuccess;
}

}  // namespace tile
}  // namespace attn
