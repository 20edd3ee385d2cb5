// hisparse_sparse_mla_decode_noalloc: the sparse MLA decode attention for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// It is hisparse_sparse_mla_decode with its workspace -- the per-split
// partial outputs and their (max, sum) pairs -- taken from a fixed device
// array of this file instead of a caller buffer.  The array is a
// file-scope __device__ variable: every GPU the library runs on holds its
// own copy (kNoallocScratchBytes) until the process ends.  Its device
// address is looked up once per device, with that device current, when a
// handle is created there (hisparse_create); host code uses only that
// address (the variable's name is a host-side stand-in, not a device
// pointer).  The entry point makes no HIP allocation or lookup of its own.
//
// Every call on one GPU shares that GPU's array: calls that overlap in time
// on one GPU (different streams without an ordering between them) race on
// it.  Nothing in it has to start at zero: the split kernel writes every
// partial the merge kernel reads, within the same call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hisparse.h"
#include "hisparse_entry.h"

namespace {

constexpr size_t kNoallocScratchBytes = HISPARSE_NOALLOC_SCRATCH_BYTES;  // per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace hsp {

// Set-up, from hisparse_create with the new handle's device current: look up
// that device's copy of `scratch` once and keep its address.
int noalloc_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(HISPARSE_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return HISPARSE_OK;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    return set_error(HISPARSE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                     hipGetErrorString(e));
  }
  g_scratch_ptr[dev] = p;
  return HISPARSE_OK;
}

}  // namespace hsp

namespace {

// The address noalloc_setup kept for the handle's device.
int scratch_of(hisparse_t h, void** out) {
  *out = nullptr;
  const int dev = hsp::handle_device(h);
  if (dev < 0 || dev >= kMaxDevices)
    return hsp::set_error(HISPARSE_ERR_INVALID_ARG, "handle without a device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  *out = g_scratch_ptr[dev];
  if (!*out) return hsp::set_error(HISPARSE_ERR_STATE, "no scratch set up on device %d", dev);
  return HISPARSE_OK;
}

}  // namespace

extern "C" {

int hisparse_sparse_mla_decode_noalloc(hisparse_t h, hipStream_t stream, int32_t layer,
                                       const void* q, const int32_t* out_slot, int32_t num_heads,
                                       float scale, float* out, float* lse) {
  size_t need = 0;
  int rc = hisparse_mla_workspace_bytes(h, num_heads, &need);  // validates h and num_heads
  if (rc) return rc;
  if (need > kNoallocScratchBytes)
    return hsp::set_error(HISPARSE_ERR_UNSUPPORTED,
                          "attention of %d heads needs %zu bytes of workspace; the no-alloc "
                          "entry point holds %zu (use hisparse_sparse_mla_decode with a "
                          "workspace of that size)",
                          num_heads, need, kNoallocScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_of(h, &ws))) return rc;
  return hisparse_sparse_mla_decode(h, stream, layer, q, out_slot, num_heads, scale, ws, out,
                                    lse);
}

}  // extern "C"
