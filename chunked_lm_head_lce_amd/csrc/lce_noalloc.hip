// lce_forward_noalloc: the forward of include/lce.h for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). Its workspace is a file-scope device
// array of LCE_NOALLOC_SCRATCH_BYTES per GPU, held from the moment the
// library's code is loaded on that GPU until the process ends.
//
// Host code never passes the array's name to a kernel or a copy: on the host
// `scratch` is only a stand-in for the symbol. Its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and
// kept; every use goes through that address.
//
// Every call on one GPU shares that GPU's array and it keeps the previous
// call's contents: the forward clears what must start at zero (the valid
// count, the status word, the chunk sums and the tile counters) with its own
// kernels, so no call depends on an earlier one. Calls that overlap on one
// GPU (several streams or threads at once) race on the array; callers must
// order them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "lce_internal.h"

static __device__ __align__(256) unsigned char scratch[LCE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up
std::mutex g_scratch_mu;

// Device address of this device's `scratch` (looked up on first use).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LCE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return LCE_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return LCE_OK;
}

// Rows whose (max, sum-exp) partials the forward holds at once so that its
// whole workspace fits the array: 0 when every row fits in one pass, else the
// largest multiple of 256 that fits, -1 when not even 256 rows do.
int64_t fitting_group(const lce_problem* p) {
  const size_t cap = LCE_NOALLOC_SCRATCH_BYTES;
  if (lce::forward_workspace_bytes(p, 0) <= cap) return 0;
  if (lce::forward_workspace_bytes(p, 256) > cap) return -1;
  int64_t lo = 1, hi = (p->n_rows + 255) / 256;   // in tiles of 256 rows: lo fits, hi does not
  while (hi - lo > 1) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (lce::forward_workspace_bytes(p, mid * 256) <= cap) lo = mid;
    else hi = mid;
  }
  return lo * 256;
}

}  // namespace

extern "C" int lce_forward_noalloc(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                                   const int64_t* labels, float* loss, float* lse, float* chunk_loss,
                                   int64_t* n_valid, int32_t* status, hipStream_t stream) {
  if (lce::forward_workspace_bytes(p, 0) == 0)   // invalid problem: the same host checks report why
    return lce::forward_grouped(p, hidden, weight, bias, labels, loss, lse, chunk_loss, n_valid, status, nullptr,
                                0, 0, stream, nullptr);
  const int64_t group = fitting_group(p);
  if (group < 0) return LCE_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != LCE_OK) return st;
  return lce::forward_grouped(p, hidden, weight, bias, labels, loss, lse, chunk_loss, n_valid, status, ws,
                              LCE_NOALLOC_SCRATCH_BYTES, group, stream, nullptr);
}
