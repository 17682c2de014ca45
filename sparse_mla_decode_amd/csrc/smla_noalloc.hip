// smla_noalloc.hip -- smla_decode_noalloc: smla_decode for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  The partials of a split call live
// in a file-scope device array instead of a caller's workspace; the caller
// still passes q, the cache, the list and the outputs.
//
// The array is a host-side stand-in in host code: its device address is
// fetched once per device (hipGetSymbolAddress, with that device current) and
// only that address is ever passed to a kernel.  Each device holds its own
// copy until the process ends.  No call here allocates or frees memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/smla.h"

#define SMLA_API extern "C" __attribute__((visibility("default")))

static_assert(SMLA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

// The partials of every smla_decode_noalloc call on this device: part_o then
// part_lse, laid out as smla_decode's workspace.  Nothing in it needs to be
// zero at the start of a call (every slot a call reads, that call writes).
static __device__ __align__(256) unsigned char scratch[SMLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address per device, once known
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return SMLA_ERR_DEVICE;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return SMLA_ERR_DEVICE;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SMLA_OK;
}

}  // namespace

SMLA_API int smla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* topk_idx,
                                 void* out, float* lse, float scale, int nsplit, int batch,
                                 int q_len, int heads, int topk, int64_t kv_rows,
                                 void* hip_stream) {
  if (nsplit < 0 || nsplit > SMLA_MAX_NSPLIT) return SMLA_ERR_NSPLIT;
  if (nsplit == 0) {
    nsplit = smla_plan_nsplit(batch, q_len, heads, topk);
    if (nsplit < 1) return nsplit;
  }
  const size_t need = smla_workspace_bytes(batch, q_len, heads, nsplit);
  if (need > (size_t)SMLA_NOALLOC_SCRATCH_BYTES) return SMLA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_address(&ws);
    if (rc != SMLA_OK) return rc;
  }
  return smla_decode(q, kv_cache, topk_idx, out, lse, scale, nsplit, batch, q_len, heads, topk,
                     kv_rows, ws, need, hip_stream);
}
