// moe_schedule_noalloc: the schedule (histogram + scan + stable placement, route.hip) for callers
// that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). Its scratch, the per-block histograms [nblk][E] and the m-tile prefix
// [E + 1] that moe_schedule keeps in the caller's workspace, lives in a file-scope device array
// instead. Every GPU the library runs on holds its own copy of the array until the process
// ends; the host looks up each device's address once (hipGetSymbolAddress with that device
// current) and passes that address to the kernels. In host code the array's name is only a
// host-side stand-in, never a device address.
//
// Every call on a GPU shares that GPU's array and leaves its contents behind. Nothing in it has
// to start at zero: the histogram pass writes every entry of [nblk][E] and the scan pass every
// entry of the prefix before anything reads them. Calls that overlap on one GPU (two streams,
// two host threads) race on the array; callers serialise them.
#include <mutex>

#include "common.h"

namespace moe {

// 2 MiB of histograms (nblk * E <= 2^19 int32: e.g. 2^20 routes with E = 1024, or 2^22 routes
// with E = 256) after 8 KiB for the m-tile prefix (E + 1 <= 1025 int32).
constexpr int64_t kNoAllocPrefixInts = 2048;
constexpr int64_t kNoAllocHistInts = (int64_t)1 << 19;

static __device__ __align__(256) int32_t scratch[kNoAllocPrefixInts + kNoAllocHistInts];

constexpr int kMaxNoAllocDevices = 64;
static std::mutex g_scratch_mutex;
static int32_t* g_scratch_addr[kMaxNoAllocDevices];   // device address of `scratch` per device

// The current device's address of `scratch`, looked up on the first call on that device.
static int scratch_on_current_device(int32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxNoAllocDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    g_scratch_addr[dev] = (int32_t*)ptr;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_schedule_noalloc(const moe_problem* p, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* inv_perm, int32_t* error_word, hipStream_t stream) {
  int st = validate_routing(p);
  if (st) return st;
  if (!topk_idx || !counts || !offsets || !perm || !inv_perm || !error_word) return MOE_ERR_INVALID_ARG;
  const int64_t n = (int64_t)p->T * p->K;
  const int64_t nblk = (n + kRouteRowsPerBlock - 1) / kRouteRowsPerBlock;
  if (nblk * p->E > kNoAllocHistInts || p->E + 1 > kNoAllocPrefixInts) return MOE_ERR_UNSUPPORTED;
  int32_t* s = nullptr;
  if ((st = scratch_on_current_device(&s))) return st;
  return launch_schedule(topk_idx, p->T, p->K, p->E, counts, offsets, perm, inv_perm, s + kNoAllocPrefixInts, s,
                         error_word, stream);
}

}  // extern "C"
