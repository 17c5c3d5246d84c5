// Work items of a variable-length batch ("Flash Attention 3：让 GPU 跑满的注意力
// 计算", §5.2: sequences packed along the token axis, described by cu_seqlens
// prefix sums, no padding).
//
// Each sequence's rows are cut into tiles of R rows that restart at the
// sequence's first row, so no tile mixes two sequences.  Tile j of sequence
// s gets the slot
//     slot(s, j) = floor(a_s / R) + s + j,   0 <= j < ceil(L_s / R),
// with a_s = cu[s] clamped into [0, N] and L_s the sequence's length.  The
// slot ranges of consecutive sequences do not overlap (floor(a / R) +
// ceil(L / R) <= floor((a + L) / R) + 1) and all lie below floor(N / R) + B,
// a bound the host knows without reading cu_seqlens (which is device
// memory).  A workgroup finds the sequence of its slot with one round of
// vector loads: lane l reads sequence base + l, and as first slots grow with
// s, the owner can only be the last lane whose first slot is <= the slot,
// found by a ballot.  Past 64 sequences a binary search over blocks of 64 (scalar
// loads) picks `base` first.  A slot no tile owns exits at once (at most
// B + 1 per head).  The same numbering places the per-tile fp8 scales of a
// packed batch (R = 128), so a kernel finds the scales of a sequence without
// summing over the sequences before it.
#pragma once

#include <atomic>

#include "attn_device.h"

namespace attn {
namespace sched {

// First slot of the sequence whose rows start at a (clamped) and whose index
// is s.
template <int R>
__device__ __forceinline__ int first_slot(int a, int s) {
  return a / R + s;
}

struct SlotTile {
  int seq;     // sequence index
  int j;       // tile index within the sequence
  int a, e;    // the sequence's rows [a, e) in the tiled array
  int oa, oe;  // its rows [oa, oe) in the other array (keys of a query tile, ...)
};

// The tile that owns `slot` of a batch of B sequences over N rows (cu: device
// array of B + 1 prefix sums), with the same sequence's rows in a second
// array (cu_o over N_o rows); false if no tile owns the slot.  Prefix sums are
// clamped as the kernels clamp them: a = cu[s] into [0, N], e = cu[s + 1]
// into [a, N].  Call with the whole wave active and wave-uniform arguments.
template <int R>
__device__ __forceinline__ bool slot_tile(const int32_t* cu, int B, int N, const int32_t* cu_o, int N_o, int slot,
                                          SlotTile& t) {
  int base = 0;
  if (B > 64) {
    // largest block c with first_slot(a_{64c}, 64c) <= slot
    int lo = 0, hi = (B + 63) / 64;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (first_slot<R>(min(max(load_uniform(cu, 64 * mid), 0), N), 64 * mid) <= slot)
        lo = mid;
      else
        hi = mid;
    }
    base = 64 * lo;
  }
  const int s = base + __lane_id();
  const int i0 = min(s, B), i1 = min(s + 1, B);  // in bounds: cu has B + 1 entries
  const int x = cu[i0], y = cu[i1], ox = cu_o[i0], oy = cu_o[i1];
  const int a = min(max(x, 0), N);
  const uint64_t below = __ballot(s < B && first_slot<R>(a, s) <= slot);
  if (below == 0) return false;
  const int l = 63 - __builtin_clzll(below);  // the last such lane
  t.seq = base + l;
  t.a = __builtin_amdgcn_readlane(a, l);
  t.e = min(max(__builtin_amdgcn_readlane(y, l), t.a), N);
  t.oa = min(max(__builtin_amdgcn_readlane(ox, l), 0), N_o);
  t.oe = min(max(__builtin_amdgcn_readlane(oy, l), t.oa), N_o);
  t.j = slot - first_slot<R>(t.a, t.seq);  // >= 0 by the ballot
  return t.j < (t.e - t.a + R - 1) / R;
}

// Work index t of a launch over the R-row tiles of a packed batch -> its
// tile (the rows as in slot_tile); false if t names no tile.  Up to
// kScanSeqs sequences the tiles are numbered sequence after sequence and
// found by a scan of the prefix sums (one round of scalar loads per
// sequence passed; the long first sequences hold most tiles, and this is
// the shortest start-up path measured for a few sequences); past that, t
// is a slot (slot_tile: one round of vector loads after an O(log B) search).
// Both numberings stay below ceil(N / R) + B.
constexpr int kScanSeqs = 16;

template <int R>
__device__ __forceinline__ bool find_tile(const int32_t* cu, int B, int N, const int32_t* cu_o, int N_o, int t,
                                          SlotTile& out) {
  if (B > kScanSeqs) return slot_tile<R>(cu, B, N, cu_o, N_o, t, out);
  int acc = 0;
  for (int s = 0; s < B; ++s) {
    const int a = min(max(cu[s], 0), N);
    const int e = min(max(cu[s + 1], a), N);
    const int nt = (e - a + R - 1) / R;
    if (t < acc + nt) {
      out.seq = s;
      out.j = t - acc;
      out.a = a;
      out.e = e;
      out.oa = min(max(cu_o[s], 0), N_o);
      out.oe = min(max(cu_o[s + 1], out.oa), N_o);
      return true;
    }
    acc += nt;
  }
  return false;
}

// ---------------------------------------------------------------------------
// Persistent grids: CUs x (workgroups one CU holds) workgroups that take
// work items from one queue per XCD until it is empty.  Each queue serves
// the XCD's contiguous range of items (the ranges xcd_remap gives the
// dispatcher), so the order of the items and their L2 locality stay the
// same.  An item that owns no tile then costs a lookup and a barrier
// instead of a workgroup launch.
//
// A queue slot holds one counter per XCD and a count of finished
// workgroups, each on its own 256-byte line (packed counters measured 2 %
// slower).  The slots are zero when the code object loads (each kernel
// file holds its own array); the last workgroup of a launch clears its slot
// again, so a launch needs neither a workspace nor a reset.  Each stream
// has a slot of its own (queue_slot), as launches on one stream never
// overlap.
constexpr int kQueueSlots = 256;
constexpr int kQueueStride = 64;                // unsigned ints between counters
constexpr int kQueueWords = 9 * kQueueStride;  // one slot

// f(item) for the items this workgroup takes from slot q.  Lane 0 claims
// the next item with a device atomic before running the current one and the
// claim is read after it, so its latency overlaps the item.  f must leave
// LDS free for the next item (a barrier separates the items).
template <typename F>
__device__ __forceinline__ void persistent_items(unsigned int* q, int n_work, F&& f) {
  __shared__ int next_item[2];
  const int x = blockIdx.x & 7;  // the XCD (workgroups are dealt round-robin)
  const int per = n_work >> 3, rem = n_work & 7;
  const int lo = x * per + min(x, rem), cnt = per + (x < rem ? 1 : 0);
  unsigned int* head = q + x * kQueueStride;
  if (threadIdx.x == 0) {
    const unsigned t = atomicAdd(head, 1u);
    next_item[0] = t < (unsigned)cnt ? lo + (int)t : -1;
  }
  int buf = 0;
  for (;;) {
    __syncthreads();
    const int item = next_item[buf];
    if (item < 0) break;
    unsigned t_next = 0;
    if (threadIdx.x == 0) t_next = atomicAdd(head, 1u);
    f(item);
    if (threadIdx.x == 0) next_item[buf ^ 1] = t_next < (unsigned)cnt ? lo + (int)t_next : -1;
    buf ^= 1;
  }
  if (threadIdx.x == 0) {
    // every claim of this workgroup has returned; the last one out clears the slot
    __threadfence();
    if (atomicAdd(q + 8 * kQueueStride, 1u) == gridDim.x - 1) {
      __threadfence();
      for (int y = 0; y < 9; ++y) atomicExch(q + y * kQueueStride, 0u);
    }
  }
}

}  // namespace sched

namespace tile {
hipError_t device_cu_count(int* cus);
}

namespace sched {

// The queue slot of the launches on stream st (attn_fwd.hip).  False, and
// the launch uses the dispatcher: the stream is being captured (the replays
// of a graph would share the slot recorded at capture), it is the per-thread
// default stream (one handle for the streams of many threads), or
// kQueueSlots streams already hold a slot.
bool queue_slot(hipStream_t st, int* slot);

// Workgroups of a persistent launch of kern: CUs x the workgroups one CU
// holds (asked of the runtime once; per_cu caches it per kernel), at most
// n_work.
inline hipError_t persistent_grid(const void* kern, int threads, int lds_bytes, int n_work,
                                  std::atomic<int>& per_cu_cache, unsigned* grid) {
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds_bytes);
    if (e != hipSuccess) return e;
    per_cu = per_cu < 1 ? 1 : per_cu;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  int cus = 0;
  const hipError_t e = tile::device_cu_count(&cus);
  if (e != hipSuccess) return e;
  const int64_t g = (int64_t)cus * per_cu;
  *grid = (unsigned)(g < n_work ? g : n_work);
  return hipSuccess;
}

}  // namespace sched
}  // namespace attn
