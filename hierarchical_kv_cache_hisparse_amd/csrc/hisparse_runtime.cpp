// Host runtime of libhisparse: the C ABI declared in include/hisparse.h.
//
// It validates shapes, owns the handle (events, a device copy of the host
// history pointers, per-layer prefetch buffers) and enqueues the gfx950
// kernels.  resolve / prefetch / append / load_window / reset never
// synchronize, allocate or read device memory, so a caller can capture them
// into a HIP graph ("HiSparse: Scaling Sparse-Attention Decoding with
// Hierarchical KV Cache Management", Abstract: resolution runs inside the
// decode graph; "Hybrid HiSparse", Timeline: the kernel is graph-capturable).
#include <hip/hip_runtime_api.h>
#include <linux/mempolicy.h>
#include <sys/syscall.h>
#include <unistd.h>

#include <cerrno>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "hisparse.h"
#include "hisparse_entry.h"
#include "hisparse_internal.h"
#include "hisparse_mla_internal.h"
#include "hisparse_topk_internal.h"

using namespace hsp;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HISPARSE_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

#define HIP_TRY(call)                           \
  do {                                          \
    hipError_t e_ = (call);                     \
    if (e_ != hipSuccess) return hip_fail(e_, #call); \
  } while (0)

constexpr int kMaxNumaNodes = 1024;  // node masks handed to the memory-policy calls

constexpr uint32_t kKnownFlags =
    HISPARSE_NO_IO | HISPARSE_DEBUG_VALIDATE | HISPARSE_SERIALIZE_PREFETCH;

int validate_config(const hisparse_config* c) {
  if (!c) return fail(HISPARSE_ERR_INVALID_ARG, "config is NULL");
  if (c->num_requests < 1 || c->num_layers < 1)
    return fail(HISPARSE_ERR_INVALID_ARG, "num_requests and num_layers must be >= 1");
  if (c->num_requests > kMaxRequests)
    return fail(HISPARSE_ERR_UNSUPPORTED, "num_requests %d exceeds %d", c->num_requests,
                kMaxRequests);
  if (c->max_positions < 1 || c->max_positions >= (int64_t(1) << 31))
    return fail(HISPARSE_ERR_INVALID_ARG, "max_positions must be in [1, 2^31)");
  if (c->row_bytes <= 0 || c->row_bytes % 16 != 0)
    return fail(HISPARSE_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 16");
  if (c->top_k < 1) return fail(HISPARSE_ERR_INVALID_ARG, "top_k must be >= 1");
  if (c->cache_slots < c->top_k)
    return fail(HISPARSE_ERR_INVALID_ARG, "cache_slots (%d) must be >= top_k (%d)",
                c->cache_slots, c->top_k);
  if (c->resident_window < 0)
    return fail(HISPARSE_ERR_INVALID_ARG, "resident_window must be >= 0");
  if (c->flags & ~kKnownFlags) return fail(HISPARSE_ERR_INVALID_ARG, "unknown flags 0x%x", c->flags);
  if (c->top_k > kMaxTopK)
    return fail(HISPARSE_ERR_UNSUPPORTED, "top_k %d exceeds %d", c->top_k, kMaxTopK);
  if (c->cache_slots > kMaxSlots)
    return fail(HISPARSE_ERR_UNSUPPORTED, "cache_slots %d exceeds %d", c->cache_slots, kMaxSlots);
  if ((int64_t)c->cache_slots + c->resident_window >= (int64_t(1) << 31))
    return fail(HISPARSE_ERR_INVALID_ARG, "cache_slots + resident_window too large");
  // (C+R) * row_bytes must fit the 32-bit byte counters of one slot row set
  const double per_stream = (double)(c->cache_slots + c->resident_window) * c->row_bytes;
  if (per_stream * c->num_layers * c->num_requests > 9.0e18)
    return fail(HISPARSE_ERR_INVALID_ARG, "cache size overflows");
  if ((int64_t)c->top_k * c->row_bytes >= (int64_t(1) << 31))
    return fail(HISPARSE_ERR_UNSUPPORTED, "top_k * row_bytes must be < 2^31");
  const ResolveShape sh =
      resolve_shape(c->top_k, c->cache_slots, (c->flags & HISPARSE_DEBUG_VALIDATE) != 0);
  if (sh.items == 0 || sh.lds_bytes > kMaxLdsBytes)
    return fail(HISPARSE_ERR_UNSUPPORTED,
                "C=%d, k=%d need %zu bytes of LDS per workgroup (limit %zu)", c->cache_slots,
                c->top_k, sh.lds_bytes, kMaxLdsBytes);
  return HISPARSE_OK;
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

struct TimedCall {
  hipEvent_t e0, e1, e2, e3;  // resolve kernel start / end, fetch kernel start / end
  bool fetched;
};

}  // namespace

namespace hsp {
int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}
}  // namespace hsp

struct hisparse {
  hisparse_config cfg;
  hisparse_meta_layout lay;
  int device = 0;
  StreamView view{};
  uint8_t** d_host = nullptr;    // [L*B] host-history pointers, device copy
  int32_t* pf_out = nullptr;     // [L][B][k] prefetched slot maps
  int32_t* pf_sel = nullptr;     // [L][B][k] prefetched selections
  std::vector<uint8_t> pending;  // per layer: a prefetch waits to be joined
  std::vector<int32_t*> pf_dst;      // per layer: where the pending prefetch writes its map
  std::vector<const int32_t*> pf_src;  // per layer: the selections it was given
  std::vector<hipEvent_t> ev_fork, ev_done;
  int fetch_grid_x = 64;  // fetch kernel workgroups
  size_t lds_max = 0;     // LDS bytes per workgroup of the device
  // timing of eager calls
  bool timing = false;
  std::vector<TimedCall> pool;
  size_t pool_used = 0;
  hisparse_timing totals{};
};

namespace hsp {
int handle_device(const hisparse* h) { return h ? h->device : -1; }
}  // namespace hsp

namespace {

int fold_timing(hisparse* h) {
  for (size_t i = 0; i < h->pool_used; ++i) {
    TimedCall& c = h->pool[i];
    HIP_TRY(hipEventSynchronize(c.fetched ? c.e3 : c.e1));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, c.e0, c.e1));
    h->totals.resolve_ms += ms;
    h->totals.resolve_launches += 1;
    if (c.fetched) {
      HIP_TRY(hipEventElapsedTime(&ms, c.e2, c.e3));
      h->totals.fetch_ms += ms;
      h->totals.fetch_launches += 1;
    }
  }
  h->pool_used = 0;
  return HISPARSE_OK;
}

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return false;
  return st != hipStreamCaptureStatusNone;
}

// resolve kernel (+ fetch unless NO_IO) of one layer on one stream
int enqueue_resolve(hisparse* h, hipStream_t s, const int32_t* sel, const int32_t* ctx_len,
                    int layer, int32_t* out, int32_t* sel_copy, int multi_entries = 0,
                    const uint8_t* app_rows = nullptr, const int32_t* app_pos = nullptr) {
  const bool io = !(h->cfg.flags & HISPARSE_NO_IO);
  TimedCall* tc = nullptr;
  if (h->timing && !capturing(s)) {
    if (h->pool_used == h->pool.size()) {
      int rc = fold_timing(h);
      if (rc) return rc;
    }
    tc = &h->pool[h->pool_used++];
    tc->fetched = io && !h->view.fuse_fetch;
  }
  // timed calls: events attached to each kernel's own dispatch
  HIP_TRY(launch_resolve(h->view, s, layer, sel, ctx_len, out, sel_copy, multi_entries, app_rows,
                         app_pos, tc ? tc->e0 : nullptr, tc ? tc->e1 : nullptr));
  if (io && !h->view.fuse_fetch)
    HIP_TRY(launch_fetch(h->view, s, layer, h->fetch_grid_x, tc ? tc->e2 : nullptr,
                         tc ? tc->e3 : nullptr));
  return HISPARSE_OK;
}

void release(hisparse* h) {
  if (!h) return;
  for (auto e : h->ev_fork) if (e) (void)hipEventDestroy(e);
  for (auto e : h->ev_done) if (e) (void)hipEventDestroy(e);
  for (auto& c : h->pool) {
    (void)hipEventDestroy(c.e0);
    (void)hipEventDestroy(c.e1);
    (void)hipEventDestroy(c.e2);
    (void)hipEventDestroy(c.e3);
  }
  if (h->d_host) (void)hipFree(h->d_host);
  if (h->pf_out) (void)hipFree(h->pf_out);
  if (h->pf_sel) (void)hipFree(h->pf_sel);
  delete h;
}

// true when [a, a + na) and [b, b + nb) share a byte
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// out_slot is written while sel and ctx_len are still being read
int check_no_overlap(const hisparse* h, const int32_t* sel, size_t sel_entries,
                     const int32_t* ctx_len, const int32_t* out) {
  const size_t B = (size_t)h->cfg.num_requests;
  const size_t out_bytes = sizeof(int32_t) * sel_entries;
  if (overlaps(out, out_bytes, sel, sizeof(int32_t) * sel_entries) ||
      overlaps(out, out_bytes, ctx_len, sizeof(int32_t) * B))
    return fail(HISPARSE_ERR_INVALID_ARG, "out_slot overlaps sel or ctx_len");
  return HISPARSE_OK;
}

// the host-side checks of a multi-query resolve
int check_multi(const hisparse* h, const int32_t* sel, int32_t queries, int32_t per_query,
                const int32_t* ctx_len, int32_t layer, const int32_t* out_slot) {
  if (!h) return fail(HISPARSE_ERR_INVALID_ARG, "handle is NULL");
  if (!sel || !ctx_len || !out_slot)
    return fail(HISPARSE_ERR_INVALID_ARG, "sel, ctx_len and out_slot must not be NULL");
  if (layer < 0 || layer >= h->cfg.num_layers)
    return fail(HISPARSE_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, h->cfg.num_layers);
  if (queries < 1 || per_query < 1 || (int64_t)queries * per_query > h->cfg.top_k)
    return fail(HISPARSE_ERR_INVALID_ARG,
                "queries (%d) x per_query (%d) must be in [1, top_k = %d]", queries, per_query,
                h->cfg.top_k);
  if (h->pending[layer])
    return fail(HISPARSE_ERR_STATE, "layer %d has a pending prefetch: join it with hisparse_resolve",
                layer);
  const int ke = queries * per_query;
  if (int rc = check_no_overlap(h, sel, (size_t)h->cfg.num_requests * ke, ctx_len, out_slot))
    return rc;
  const ResolveShape sh = resolve_shape(h->cfg.top_k, h->cfg.cache_slots,
                                        (h->cfg.flags & HISPARSE_DEBUG_VALIDATE) != 0, ke);
  if (sh.lds_bytes > h->lds_max)
    return fail(HISPARSE_ERR_UNSUPPORTED,
                "C=%d with %d entries per request needs %zu bytes of LDS; the device has %zu",
                h->cfg.cache_slots, ke, sh.lds_bytes, h->lds_max);
  return HISPARSE_OK;
}

int check_device_buffer(const void* p, const char* name) {
  if (!p) return fail(HISPARSE_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 256 != 0)
    return fail(HISPARSE_ERR_INVALID_ARG, "%s must be 256-byte aligned", name);
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess || attr.type != hipMemoryTypeDevice) {
    (void)hipGetLastError();
    return fail(HISPARSE_ERR_INVALID_ARG, "%s is not device memory", name);
  }
  return HISPARSE_OK;
}

}  // namespace

extern "C" {

int hisparse_workspace_bytes(const hisparse_config* cfg, size_t* cache_bytes, size_t* meta_bytes) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (cache_bytes)
    *cache_bytes = (size_t)cfg->num_layers * cfg->num_requests *
                   ((size_t)cfg->cache_slots + cfg->resident_window) * cfg->row_bytes;
  if (meta_bytes) *meta_bytes = meta_layout(*cfg).total_bytes;
  return HISPARSE_OK;
}

int hisparse_meta_layout_of(const hisparse_config* cfg, hisparse_meta_layout* out) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!out) return fail(HISPARSE_ERR_INVALID_ARG, "out is NULL");
  *out = meta_layout(*cfg);
  return HISPARSE_OK;
}

int hisparse_device_numa_node(int* node) {
  if (!node) return fail(HISPARSE_ERR_INVALID_ARG, "node is NULL");
  *node = -1;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  int id = -1;
  if (hipDeviceGetAttribute(&id, hipDeviceAttributeHostNumaId, dev) != hipSuccess) {
    (void)hipGetLastError();
    id = -1;
  }
  *node = id >= 0 ? id : -1;
  return HISPARSE_OK;
}

int hisparse_host_numa_node(const void* host_ptr, int* node) {
  if (!host_ptr || !node) return fail(HISPARSE_ERR_INVALID_ARG, "NULL argument");
  *node = -1;
  int n = -1;
  // the node of the page holding host_ptr (MPOL_F_NODE | MPOL_F_ADDR)
  if (syscall(SYS_get_mempolicy, &n, nullptr, 0UL, const_cast<void*>(host_ptr),
              (unsigned long)(MPOL_F_NODE | MPOL_F_ADDR)) == 0) {
    *node = n;
    return HISPARSE_OK;
  }
  // Pinned memory from the GPU driver is a device-file mapping whose pages
  // the kernel does not place-query (EFAULT).  On a host with one NUMA node
  // every page is on that node; otherwise the placement is unknown (-1).
  int count = 0, only = -1;
  for (int i = 0; i < kMaxNumaNodes; ++i) {
    char path[64];
    snprintf(path, sizeof(path), "/sys/devices/system/node/node%d", i);
    if (access(path, F_OK) == 0) {
      ++count;
      only = i;
    }
  }
  if (count == 1) *node = only;
  return HISPARSE_OK;
}

int hisparse_host_alloc(size_t bytes, int numa_node, uint32_t flags, void** host_ptr) {
  if (!host_ptr) return fail(HISPARSE_ERR_INVALID_ARG, "host_ptr is NULL");
  *host_ptr = nullptr;
  if (bytes == 0) return fail(HISPARSE_ERR_INVALID_ARG, "bytes is 0");
  if (flags & ~HISPARSE_HOST_NONCOHERENT)
    return fail(HISPARSE_ERR_INVALID_ARG, "unknown host flags 0x%x", flags);
  if (numa_node < HISPARSE_NUMA_DEFAULT || numa_node >= kMaxNumaNodes)
    return fail(HISPARSE_ERR_INVALID_ARG, "numa_node %d outside [%d, %d)", numa_node,
                HISPARSE_NUMA_DEFAULT, kMaxNumaNodes);
  int node = numa_node;
  if (node == HISPARSE_NUMA_DEVICE) {
    int rc = hisparse_device_numa_node(&node);
    if (rc) return rc;  // node stays -1 when the device reports none
  }
  unsigned hf = hipHostMallocMapped | hipHostMallocPortable |
                ((flags & HISPARSE_HOST_NONCOHERENT) ? hipHostMallocNonCoherent
                                                     : hipHostMallocCoherent);
  // Placement: bind this thread's memory policy to `node` around the
  // allocation, and tell HIP to follow that policy (hipHostMallocNumaUser);
  // the previous policy is restored afterwards.
  // A node asked for explicitly must be available; the device's own node is
  // taken when the process may allocate there, else the allocation falls back
  // to the process's policy (hisparse_host_numa_node tells where it landed).
  unsigned long old_mask[kMaxNumaNodes / 64] = {0};
  int old_mode = MPOL_DEFAULT;
  bool bind = node >= 0;
  if (bind) {
    if (syscall(SYS_get_mempolicy, &old_mode, old_mask, (unsigned long)kMaxNumaNodes, nullptr,
                0UL) != 0)
      return fail(HISPARSE_ERR_INVALID_ARG, "get_mempolicy failed: %s", strerror(errno));
    unsigned long mask[kMaxNumaNodes / 64] = {0};
    mask[node / 64] = 1UL << (node % 64);
    if (syscall(SYS_set_mempolicy, MPOL_BIND, mask, (unsigned long)kMaxNumaNodes) != 0) {
      if (numa_node != HISPARSE_NUMA_DEVICE)
        return fail(HISPARSE_ERR_INVALID_ARG, "cannot bind host memory to NUMA node %d: %s",
                    node, strerror(errno));
      bind = false;
    }
  }
  if (bind) hf |= hipHostMallocNumaUser;
  hipError_t e = hipHostMalloc(host_ptr, bytes, hf);
  if (bind) {
    const bool had_mask = old_mode != MPOL_DEFAULT && old_mode != MPOL_LOCAL;
    (void)syscall(SYS_set_mempolicy, old_mode, had_mask ? old_mask : nullptr,
                  had_mask ? (unsigned long)kMaxNumaNodes : 0UL);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *host_ptr = nullptr;
    return fail(HISPARSE_ERR_OOM, "hipHostMalloc of %zu bytes (NUMA node %d) failed: %s", bytes,
                node, hipGetErrorString(e));
  }
  return HISPARSE_OK;
}

int hisparse_host_free(void* host_ptr) {
  if (!host_ptr) return HISPARSE_OK;
  HIP_TRY(hipHostFree(host_ptr));
  return HISPARSE_OK;
}

int hisparse_create(const hisparse_config* cfg, void* const* host_rows, void* device_cache,
                    void* device_meta, hisparse_t* out) {
  if (!out) return fail(HISPARSE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!host_rows) return fail(HISPARSE_ERR_INVALID_ARG, "host_rows is NULL");
  if ((rc = check_device_buffer(device_cache, "device_cache"))) return rc;
  if ((rc = check_device_buffer(device_meta, "device_meta"))) return rc;
  const int L = cfg->num_layers, B = cfg->num_requests;
  std::vector<uint8_t*> dev_host((size_t)L * B);
  for (int i = 0; i < L * B; ++i) {
    if (!host_rows[i]) return fail(HISPARSE_ERR_INVALID_ARG, "host_rows[%d] is NULL", i);
    void* dp = nullptr;
    if (hipHostGetDevicePointer(&dp, host_rows[i], 0) != hipSuccess || !dp) {
      (void)hipGetLastError();
      return fail(HISPARSE_ERR_INVALID_ARG,
                  "host_rows[%d] is not pinned, device-mapped host memory", i);
    }
    dev_host[i] = static_cast<uint8_t*>(dp);
  }

  hisparse* h = new (std::nothrow) hisparse();
  if (!h) return fail(HISPARSE_ERR_OOM, "handle allocation failed");
  h->cfg = *cfg;
  h->lay = meta_layout(*cfg);
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) { release(h); return hip_fail(e, "hipGetDevice"); }
  {
    int lds_max = 0;
    e = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, h->device);
    if (e != hipSuccess) { release(h); return hip_fail(e, "hipDeviceGetAttribute"); }
    const ResolveShape sh =
        resolve_shape(cfg->top_k, cfg->cache_slots, (cfg->flags & HISPARSE_DEBUG_VALIDATE) != 0);
    h->lds_max = (size_t)lds_max;
    if (sh.lds_bytes > (size_t)lds_max) {
      release(h);
      return fail(HISPARSE_ERR_UNSUPPORTED, "C=%d, k=%d need %zu bytes of LDS; the device has %d",
                  cfg->cache_slots, cfg->top_k, sh.lds_bytes, lds_max);
    }
  }
  if (int rc2 = noalloc_setup(h->device)) {
    release(h);
    return rc2;
  }
  h->pending.assign(L, 0);
  h->pf_dst.assign(L, nullptr);
  h->pf_src.assign(L, nullptr);
  h->ev_fork.assign(L, nullptr);
  h->ev_done.assign(L, nullptr);
  const size_t map_bytes = sizeof(int32_t) * (size_t)L * B * cfg->top_k;
  if (hipMalloc(reinterpret_cast<void**>(&h->d_host), sizeof(uint8_t*) * L * B) != hipSuccess ||
      hipMalloc(reinterpret_cast<void**>(&h->pf_out), map_bytes) != hipSuccess ||
      hipMalloc(reinterpret_cast<void**>(&h->pf_sel), map_bytes) != hipSuccess) {
    (void)hipGetLastError();
    release(h);
    return fail(HISPARSE_ERR_OOM, "device allocation of handle buffers failed");
  }
  for (int l = 0; l < L; ++l) {
    if (hipEventCreateWithFlags(&h->ev_fork[l], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&h->ev_done[l], hipEventDisableTiming) != hipSuccess) {
      release(h);
      return fail(HISPARSE_ERR_HIP, "event creation failed");
    }
  }
  e = hipMemcpy(h->d_host, dev_host.data(), sizeof(uint8_t*) * L * B, hipMemcpyHostToDevice);
  if (e != hipSuccess) { release(h); return hip_fail(e, "hipMemcpy(host pointers)"); }

  StreamView& v = h->view;
  v.meta = static_cast<uint8_t*>(device_meta);
  v.cache = static_cast<uint8_t*>(device_cache);
  v.host = h->d_host;
  v.stream_stride = (int64_t)h->lay.stream_stride;
  v.stream_base = (int64_t)h->lay.stream_base;
  v.off_hdr = (int64_t)h->lay.hdr;
  v.off_pos2slot = (int64_t)h->lay.pos2slot;
  v.off_slot2pos = (int64_t)h->lay.slot2pos;
  v.off_last_use = (int64_t)h->lay.last_use;
  v.off_order = (int64_t)h->lay.lru_order;
  v.off_evict = (int64_t)h->lay.evict_log;
  v.off_miss = (int64_t)h->lay.miss_list;
  v.row_bytes = cfg->row_bytes;
  v.B = B;
  v.L = L;
  v.C = cfg->cache_slots;
  v.R = cfg->resident_window;
  v.k = cfg->top_k;
  v.l_cap = (int32_t)cfg->max_positions;
  v.flags = cfg->flags;
  v.r_magic = div_magic((uint32_t)cfg->resident_window);
  v.cpr_magic = div_magic((uint32_t)(cfg->row_bytes / 16));

  // Miss fetch.  One CU pulls ~12 GB/s from pinned host memory and ~8 CUs
  // saturate a PCIe Gen5 x16 link, so with >= 8 streams per layer call the
  // resolve workgroups copy their own misses (no second launch, copies start
  // as soon as the victims are known); with fewer, a separate kernel fans the
  // copies out over ~64 workgroups.  HISPARSE_FETCH_MODE=fused|split forces
  // a mode; HISPARSE_FETCH_WORKGROUPS sets the fan-out.
  const char* mode = getenv("HISPARSE_FETCH_MODE");
  if (mode && !strcmp(mode, "fused")) v.fuse_fetch = 1;
  else if (mode && !strcmp(mode, "split")) v.fuse_fetch = 0;
  else v.fuse_fetch = B >= 8 ? 1 : 0;
  // The fetch kernel indexes a layer call's chunks (B * k * row_bytes/16 at
  // most) with 32-bit counters and rounds the count up to a multiple of its
  // grid; past 2^31 chunks only the fused copy (per-stream counts) is used.
  if (!v.fuse_fetch && (int64_t)B * cfg->top_k * (cfg->row_bytes / 16) >= (int64_t(1) << 31))
    v.fuse_fetch = 1;
  const int wgs = env_int("HISPARSE_FETCH_WORKGROUPS", 64);
  h->fetch_grid_x = wgs > 1 ? wgs : 1;

  e = launch_init(v, nullptr, -1, -1, true);
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) { release(h); return hip_fail(e, "metadata initialisation"); }
  *out = h;
  return HISPARSE_OK;
}

int hisparse_destroy(hisparse_t h) {
  if (!h) return HISPARSE_OK;
  (void)hipDeviceSynchronize();
  release(h);
  return HISPARSE_OK;
}

int hisparse_resolve(hisparse_t h, hipStream_t stream, const int32_t* sel, const int32_t* ctx_len,
                     int32_t layer, int32_t* out_slot) {
  if (!h) return fail(HISPARSE_ERR_INVALID_ARG, "handle is NULL");
  if (!sel || !ctx_len || !out_slot)
    return fail(HISPARSE_ERR_INVALID_ARG, "sel, ctx_len and out_slot must not be NULL");
  if (layer < 0 || layer >= h->cfg.num_layers)
    return fail(HISPARSE_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, h->cfg.num_layers);
  if (int rc = check_no_overlap(h, sel, (size_t)h->cfg.num_requests * h->cfg.top_k, ctx_len,
                                out_slot))
    return rc;
  if (h->pending[layer]) {
    // join the prefetch: wait for it; when it wrote this very map from these
    // very selections, that is all; otherwise a kernel copies its map here
    // and compares the selections with the ones it resolved
    HIP_TRY(hipStreamWaitEvent(stream, h->ev_done[layer], 0));
    const bool same = out_slot == h->pf_dst[layer] && sel == h->pf_src[layer] &&
                      !(h->cfg.flags & HISPARSE_DEBUG_VALIDATE);
    if (!same) {
      const size_t off = (size_t)layer * h->cfg.num_requests * h->cfg.top_k;
      HIP_TRY(launch_prefetch_join(h->view, stream, sel, h->pf_sel + off, h->pf_dst[layer],
                                   out_slot));
    }
    h->pending[layer] = 0;
    return HISPARSE_OK;
  }
  return enqueue_resolve(h, stream, sel, ctx_len, layer, out_slot, nullptr);
}

int hisparse_resolve_multi(hisparse_t h, hipStream_t stream, const int32_t* sel,
                           int32_t queries, int32_t per_query, const int32_t* ctx_len,
                           int32_t layer, int32_t* out_slot) {
  int rc = check_multi(h, sel, queries, per_query, ctx_len, layer, out_slot);
  if (rc) return rc;
  return enqueue_resolve(h, stream, sel, ctx_len, layer, out_slot, nullptr, queries * per_query);
}

int hisparse_prefetch(hisparse_t h, hipStream_t main_stream, hipStream_t side_stream,
                      const int32_t* sel, const int32_t* ctx_len, int32_t layer,
                      int32_t* out_slot) {
  if (!h) return fail(HISPARSE_ERR_INVALID_ARG, "handle is NULL");
  if (!sel || !ctx_len) return fail(HISPARSE_ERR_INVALID_ARG, "sel and ctx_len must not be NULL");
  if (layer < 0 || layer >= h->cfg.num_layers)
    return fail(HISPARSE_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, h->cfg.num_layers);
  if (h->pending[layer])
    return fail(HISPARSE_ERR_STATE, "layer %d already has a pending prefetch", layer);
  if (out_slot) {
    if (int rc = check_no_overlap(h, sel, (size_t)h->cfg.num_requests * h->cfg.top_k, ctx_len,
                                  out_slot))
      return rc;
  }
  const bool serial = (h->cfg.flags & HISPARSE_SERIALIZE_PREFETCH) || side_stream == main_stream;
  hipStream_t s = serial ? main_stream : side_stream;
  if (!serial) {
    HIP_TRY(hipEventRecord(h->ev_fork[layer], main_stream));
    HIP_TRY(hipStreamWaitEvent(side_stream, h->ev_fork[layer], 0));
  }
  const size_t off = (size_t)layer * h->cfg.num_requests * h->cfg.top_k;
  int32_t* dst = out_slot ? out_slot : h->pf_out + off;
  int rc = enqueue_resolve(h, s, sel, ctx_len, layer, dst, h->pf_sel + off);
  if (rc) return rc;
  HIP_TRY(hipEventRecord(h->ev_done[layer], s));
  h->pending[layer] = 1;
  h->pf_dst[layer] = dst;
  h->pf_src[layer] = sel;
  return HISPARSE_OK;
}

int hisparse_load_window(hisparse_t h, hipStream_t stream, int32_t layer, const int32_t* ctx_len) {
  if (!h || !ctx_len) return fail(HISPARSE_ERR_INVALID_ARG, "handle and ctx_len must not be NULL");
  if (layer < -1 || layer >= h->cfg.num_layers)
    return fail(HISPARSE_ERR_INVALID_ARG, "layer %d out of range", layer);
  HIP_TRY(launch_load_window(h->view, stream, layer, ctx_len));
  return HISPARSE_OK;
}

int hisparse_append(hisparse_t h, hipStream_t stream, int32_t layer, const void* rows,
                    const int32_t* pos) {
  if (!h || !rows || !pos) return fail(HISPARSE_ERR_INVALID_ARG, "NULL argument");
  if (layer < 0 || layer >= h->cfg.num_layers)
    return fail(HISPARSE_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (reinterpret_cast<uintptr_t>(rows) % 16 != 0)
    return fail(HISPARSE_ERR_INVALID_ARG, "rows must be 16-byte aligned");
  HIP_TRY(launch_append(h->view, stream, layer, static_cast<const uint8_t*>(rows), pos));
  return HISPARSE_OK;
}

int hisparse_append_resolve(hisparse_t h, hipStream_t stream, int32_t layer, const void* rows,
                            const int32_t* pos, const int32_t* sel, const int32_t* ctx_len,
                            int32_t* out_slot) {
  if (!h || !rows || !pos || !sel || !ctx_len || !out_slot)
    return fail(HISPARSE_ERR_INVALID_ARG, "NULL argument");
  if (layer < 0 || layer >= h->cfg.num_layers)
    return fail(HISPARSE_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (reinterpret_cast<uintptr_t>(rows) % 16 != 0)
    return fail(HISPARSE_ERR_INVALID_ARG, "rows must be 16-byte aligned");
  if (int rc = check_no_overlap(h, sel, (size_t)h->cfg.num_requests * h->cfg.top_k, ctx_len,
                                out_slot))
    return rc;
  if (h->cfg.resident_window == 0 && h->pending[layer])
    return fail(HISPARSE_ERR_STATE,
                "layer %d has a pending prefetch and no resident window: the prefetch may "
                "have read the appended row before it was written (append before prefetching)",
                layer);
  if (h->cfg.resident_window == 0 || h->pending[layer]) {
    // the appended position may be fetched by this resolve (no window), or the
    // layer was resolved early: the append goes first, in its own launch
    HIP_TRY(launch_append(h->view, stream, layer, static_cast<const uint8_t*>(rows), pos));
    return hisparse_resolve(h, stream, sel, ctx_len, layer, out_slot);
  }
  return enqueue_resolve(h, stream, sel, ctx_len, layer, out_slot, nullptr, 0,
                         static_cast<const uint8_t*>(rows), pos);
}

int hisparse_append_resolve_multi(hisparse_t h, hipStream_t stream, int32_t layer,
                                  const void* rows, const int32_t* pos, const int32_t* sel,
                                  int32_t queries, int32_t per_query, const int32_t* ctx_len,
                                  int32_t* out_slot) {
  if (!h || !rows || !pos) return fail(HISPARSE_ERR_INVALID_ARG, "NULL argument");
  if (layer < 0 || layer >= h->cfg.num_layers)
    return fail(HISPARSE_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (reinterpret_cast<uintptr_t>(rows) % 16 != 0)
    return fail(HISPARSE_ERR_INVALID_ARG, "rows must be 16-byte aligned");
  int rc = check_multi(h, sel, queries, per_query, ctx_len, layer, out_slot);
  if (rc) return rc;  // nothing launched
  if (h->cfg.resident_window == 0) {
    // the appended position may be fetched by this resolve: append first
    HIP_TRY(launch_append(h->view, stream, layer, static_cast<const uint8_t*>(rows), pos));
    return enqueue_resolve(h, stream, sel, ctx_len, layer, out_slot, nullptr,
                           queries * per_query);
  }
  return enqueue_resolve(h, stream, sel, ctx_len, layer, out_slot, nullptr, queries * per_query,
                         static_cast<const uint8_t*>(rows), pos);
}

int hisparse_reset(hisparse_t h, hipStream_t stream, int32_t layer, int32_t request) {
  if (!h) return fail(HISPARSE_ERR_INVALID_ARG, "handle is NULL");
  if (layer < -1 || layer >= h->cfg.num_layers || request < -1 ||
      request >= h->cfg.num_requests)
    return fail(HISPARSE_ERR_INVALID_ARG, "layer/request out of range");
  for (int l = 0; l < h->cfg.num_layers; ++l)
    if ((layer < 0 || l == layer) && h->pending[l])
      return fail(HISPARSE_ERR_STATE, "layer %d has a pending prefetch", l);
  HIP_TRY(launch_init(h->view, stream, layer, request, false));
  return HISPARSE_OK;
}

int hisparse_get_status(hisparse_t h, uint32_t* status, int clear) {
  if (!h || !status) return fail(HISPARSE_ERR_INVALID_ARG, "NULL argument");
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(status, h->view.meta + h->lay.status, sizeof(uint32_t),
                    hipMemcpyDeviceToHost));
  if (clear) {
    const uint32_t zero = 0;
    HIP_TRY(hipMemcpy(h->view.meta + h->lay.status, &zero, sizeof(uint32_t),
                      hipMemcpyHostToDevice));
  }
  return HISPARSE_OK;
}

int hisparse_set_timing(hisparse_t h, int enable) {
  if (!h) return fail(HISPARSE_ERR_INVALID_ARG, "handle is NULL");
  if (enable && h->pool.empty()) {
    const size_t n = 1024;
    h->pool.resize(n);
    for (auto& c : h->pool) {
      if (hipEventCreate(&c.e0) != hipSuccess || hipEventCreate(&c.e1) != hipSuccess ||
          hipEventCreate(&c.e2) != hipSuccess || hipEventCreate(&c.e3) != hipSuccess)
        return fail(HISPARSE_ERR_HIP, "timing event creation failed");
    }
  }
  h->timing = enable != 0;
  h->pool_used = 0;
  h->totals = hisparse_timing{};
  return HISPARSE_OK;
}

int hisparse_get_timing(hisparse_t h, hisparse_timing* out) {
  if (!h || !out) return fail(HISPARSE_ERR_INVALID_ARG, "NULL argument");
  int rc = fold_timing(h);
  if (rc) return rc;
  *out = h->totals;
  return HISPARSE_OK;
}

int hisparse_probe_host_read(hipStream_t stream, const void* host, void* device, size_t bytes,
                             int32_t workgroups) {
  if (!host || !device || bytes == 0 || bytes % 16 != 0 || workgroups < 1)
    return fail(HISPARSE_ERR_INVALID_ARG, "bad probe arguments");
  if (reinterpret_cast<uintptr_t>(host) % 16 || reinterpret_cast<uintptr_t>(device) % 16)
    return fail(HISPARSE_ERR_INVALID_ARG, "probe buffers must be 16-byte aligned");
  HIP_TRY(launch_probe_host_read(stream, host, device, bytes, workgroups));
  return HISPARSE_OK;
}

namespace {
struct MlaWorkspace {
  size_t part, ml, total;
};
MlaWorkspace mla_workspace(const MlaShape& sh) {
  MlaWorkspace w{};
  w.part = 0;
  w.ml = align256(sizeof(float) * sh.part_floats);
  w.total = w.ml + align256(sizeof(float) * sh.ml_floats);
  return w;
}
int check_mla(const hisparse* h, int32_t num_heads) {
  if (!h) return fail(HISPARSE_ERR_INVALID_ARG, "handle is NULL");
  if (num_heads < kMlaHB || num_heads % kMlaHB != 0 || num_heads > 4096)
    return fail(HISPARSE_ERR_INVALID_ARG, "num_heads must be a positive multiple of %d (<= 4096)",
                kMlaHB);
  if (h->cfg.row_bytes % (2 * kMlaDqk) != 0)
    return fail(HISPARSE_ERR_UNSUPPORTED,
                "sparse MLA attention needs rows of whole 576-value bf16 token rows "
                "(row_bytes %d is not a multiple of %d)", h->cfg.row_bytes, 2 * kMlaDqk);
  const int64_t n_tok = (int64_t)h->cfg.top_k * (h->cfg.row_bytes / (2 * kMlaDqk));
  if (n_tok >= (int64_t(1) << 30)) return fail(HISPARSE_ERR_UNSUPPORTED, "too many token rows");
  return HISPARSE_OK;
}
}  // namespace

namespace {
// queries x per_query attention rows' entries must fit a slot-map row
int check_mla_rows(const hisparse* h, int32_t queries, int32_t per_query) {
  if (queries < 1 || per_query < 1 || (int64_t)queries * per_query > h->cfg.top_k)
    return fail(HISPARSE_ERR_INVALID_ARG,
                "queries (%d) x per_query (%d) must be in [1, top_k = %d]", queries, per_query,
                h->cfg.top_k);
  if ((int64_t)h->cfg.num_requests * queries > 65535)
    return fail(HISPARSE_ERR_UNSUPPORTED, "more than 65535 attention rows");
  return HISPARSE_OK;
}

int mla_bytes(hisparse_t h, int32_t queries, int32_t per_query, int32_t num_heads,
              size_t* bytes) {
  int rc = check_mla(h, num_heads);
  if (rc) return rc;
  if ((rc = check_mla_rows(h, queries, per_query))) return rc;
  if (!bytes) return fail(HISPARSE_ERR_INVALID_ARG, "bytes is NULL");
  const MlaShape sh = mla_shape(h->cfg.num_requests * queries, num_heads, per_query,
                                h->cfg.row_bytes / (2 * kMlaDqk));
  *bytes = mla_workspace(sh).total;
  return HISPARSE_OK;
}

int mla_decode(hisparse_t h, hipStream_t stream, int32_t layer, int32_t queries,
               int32_t per_query, const void* q, const int32_t* out_slot, int32_t num_heads,
               float scale, void* workspace, float* out, float* lse) {
  int rc = check_mla(h, num_heads);
  if (rc) return rc;
  if ((rc = check_mla_rows(h, queries, per_query))) return rc;
  if (layer < 0 || layer >= h->cfg.num_layers)
    return fail(HISPARSE_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, h->cfg.num_layers);
  if (!q || !out_slot || !workspace || !out || !lse)
    return fail(HISPARSE_ERR_INVALID_ARG, "NULL argument");
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(HISPARSE_ERR_INVALID_ARG, "q must be 16-byte and workspace 256-byte aligned");
  const int B = h->cfg.num_requests;
  const int rows = B * queries;
  const int T = h->cfg.row_bytes / (2 * kMlaDqk);
  const MlaShape sh = mla_shape(rows, num_heads, per_query, T);
  const MlaWorkspace ws = mla_workspace(sh);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  MlaArgs a{};
  const int64_t stream_bytes =
      ((int64_t)h->cfg.cache_slots + h->cfg.resident_window) * h->cfg.row_bytes;
  a.cache = h->view.cache + (int64_t)layer * B * stream_bytes;
  a.stream_bytes = stream_bytes;
  a.row_bytes = h->cfg.row_bytes;
  a.slots_total = h->cfg.cache_slots + h->cfg.resident_window;
  a.T = T;
  a.k = per_query;
  a.B = rows;
  a.Qn = queries;
  a.H = num_heads;
  a.HBn = sh.HBn;
  a.S = sh.S;
  a.rows_per_split = sh.rows_per_split;
  a.scale = scale;
  a.q = static_cast<const __bf16*>(q);
  a.slots = out_slot;
  a.part = reinterpret_cast<float*>(w + ws.part);
  a.part_ml = reinterpret_cast<float*>(w + ws.ml);
  a.out = out;
  a.lse = lse;
  HIP_TRY(launch_mla(a, stream, sh.lds_bytes));
  return HISPARSE_OK;
}
}  // namespace

int hisparse_mla_workspace_bytes(hisparse_t h, int32_t num_heads, size_t* bytes) {
  if (!h) return fail(HISPARSE_ERR_INVALID_ARG, "handle is NULL");
  return mla_bytes(h, 1, h->cfg.top_k, num_heads, bytes);
}

int hisparse_sparse_mla_decode(hisparse_t h, hipStream_t stream, int32_t layer, const void* q,
                               const int32_t* out_slot, int32_t num_heads, float scale,
                               void* workspace, float* out, float* lse) {
  if (!h) return fail(HISPARSE_ERR_INVALID_ARG, "handle is NULL");
  return mla_decode(h, stream, layer, 1, h->cfg.top_k, q, out_slot, num_heads, scale, workspace,
                    out, lse);
}

int hisparse_mla_workspace_bytes_multi(hisparse_t h, int32_t queries, int32_t per_query,
                                       int32_t num_heads, size_t* bytes) {
  if (!h) return fail(HISPARSE_ERR_INVALID_ARG, "handle is NULL");
  return mla_bytes(h, queries, per_query, num_heads, bytes);
}

int hisparse_sparse_mla_decode_multi(hisparse_t h, hipStream_t stream, int32_t layer,
                                     int32_t queries, int32_t per_query, const void* q,
                                     const int32_t* out_slot, int32_t num_heads, float scale,
                                     void* workspace, float* out, float* lse) {
  if (!h) return fail(HISPARSE_ERR_INVALID_ARG, "handle is NULL");
  return mla_decode(h, stream, layer, queries, per_query, q, out_slot, num_heads, scale,
                    workspace, out, lse);
}

namespace {
int check_topk(int32_t num_rows, int64_t max_len) {
  if (num_rows < 1 || num_rows > kTopkMaxRows)
    return fail(HISPARSE_ERR_INVALID_ARG, "num_rows %d outside [1, %d]", num_rows, kTopkMaxRows);
  if (max_len < 1 || max_len > kTopkMaxLen)
    return fail(HISPARSE_ERR_INVALID_ARG, "max_len %lld outside [1, %lld]", (long long)max_len,
                (long long)kTopkMaxLen);
  return HISPARSE_OK;
}
}  // namespace

int hisparse_topk_workspace_bytes(int32_t num_rows, int64_t max_len, size_t* bytes) {
  int rc = check_topk(num_rows, max_len);
  if (rc) return rc;
  if (!bytes) return fail(HISPARSE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = topk_layout(num_rows, max_len).total;
  return HISPARSE_OK;
}

int hisparse_topk(hipStream_t stream, const float* scores, int64_t row_stride, int32_t num_rows,
                  int64_t max_len, const int32_t* ctx_len, int32_t k, void* workspace,
                  int32_t* out_sel) {
  int rc = check_topk(num_rows, max_len);
  if (rc) return rc;
  if (!scores || !ctx_len || !workspace || !out_sel)
    return fail(HISPARSE_ERR_INVALID_ARG, "NULL argument");
  if (k < 1 || k > kMaxTopK) return fail(HISPARSE_ERR_INVALID_ARG, "k %d outside [1, %d]", k, kMaxTopK);
  if (row_stride < max_len || row_stride % 4)
    return fail(HISPARSE_ERR_INVALID_ARG, "row_stride must be >= max_len and a multiple of 4");
  if (reinterpret_cast<uintptr_t>(scores) % 16 || reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(HISPARSE_ERR_INVALID_ARG, "scores must be 16-byte and workspace 256-byte aligned");
  const TopkLayout lay = topk_layout(num_rows, max_len);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  TopkArgs a{};
  a.scores = scores;
  a.row_stride = row_stride;
  a.max_len = max_len;
  a.ctx_len = ctx_len;
  a.k = k;
  a.rows = num_rows;
  a.hist = reinterpret_cast<uint32_t*>(w + lay.hist);
  a.hist2 = reinterpret_cast<uint32_t*>(w + lay.hist2);
  a.cnt = reinterpret_cast<uint32_t*>(w + lay.cnt);
  a.bitmap = reinterpret_cast<uint32_t*>(w + lay.bitmap);
  a.bm_words = lay.bm_words;
  a.cand = reinterpret_cast<uint32_t*>(w + lay.cand);
  a.out = out_sel;
  HIP_TRY(launch_topk(a, stream));
  return HISPARSE_OK;
}

const char* hisparse_strerror(int code) {
  switch (code) {
    case HISPARSE_OK: return "success";
    case HISPARSE_ERR_INVALID_ARG: return "invalid argument";
    case HISPARSE_ERR_OOM: return "out of memory";
    case HISPARSE_ERR_HIP: return "HIP runtime error";
    case HISPARSE_ERR_STATE: return "call out of order";
    case HISPARSE_ERR_UNSUPPORTED: return "unsupported shape";
    default: return "unknown error code";
  }
}

const char* hisparse_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
