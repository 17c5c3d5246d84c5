// attn_fwd_splitkv_noalloc: attn_fwd_splitkv for callers that cannot allocate
// device memory.  The per-chunk partial outputs (fp32 O and lse of every key
// chunk, which attn_fwd_splitkv takes as a caller workspace) live in a fixed
// file-scope device array, `scratch`, of kScratchBytes.  Each GPU the library
// runs on holds its own copy until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in): the
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and used from then on.
//
// The kernels write every (chunk, query row) entry they later read (a chunk a
// row cannot see writes O = 0, lse = -inf), so nothing needs clearing between
// calls.  Calls that overlap on one GPU share the array and race.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/attn.h"
#include "attn_params.h"

namespace {

constexpr size_t kScratchBytes = (size_t)ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each GPU (null: not looked up yet)

// The current device's copy of `scratch`, looked up on the first call on that
// device.  Returns hipSuccess or the lookup's error.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                        int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                                        int num_splits, void* hip_stream) {
  // attn_fwd_splitkv's checks with a stand-in (aligned, non-null) workspace,
  // then the size check: host code only, before any HIP call
  const float* stand_in = reinterpret_cast<const float*>(static_cast<uintptr_t>(256));
  const int rc = attn::validate_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, num_splits,
                                        stand_in, stand_in);
  if (rc != ATTN_OK) return rc;
  // O parts [num_splits, B, H, Nq, d] fp32 from the start of the array, then
  // the lse parts [num_splits, B, H, Nq] from the next 256-byte boundary
  const int64_t bhq = (int64_t)B * H * Nq;  // <= 2^61: B * H and Nq are checked above
  if (bhq > (int64_t)kScratchBytes) return ATTN_ERR_TOO_LARGE;
  const int64_t rows = bhq * num_splits;
  const int64_t o_bytes = (rows * d * 4 + 255) / 256 * 256;
  if (o_bytes + rows * 4 > (int64_t)kScratchBytes) return ATTN_ERR_TOO_LARGE;
  if (Nq == 0) return ATTN_OK;
  void* base = nullptr;
  if (scratch_address(&base) != hipSuccess) return ATTN_ERR_HIP;
  float* o_part = static_cast<float*>(base);
  float* lse_part = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + o_bytes);
  return attn_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, num_splits, o_part, lse_part,
                          hip_stream);
}
