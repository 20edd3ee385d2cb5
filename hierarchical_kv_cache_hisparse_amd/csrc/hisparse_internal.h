// Internal declarations shared by the host runtime and the gfx950 kernels of
// libhisparse.  Not part of the C ABI (see include/hisparse.h).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "hisparse.h"
#include "hisparse_align.h"

namespace hsp {

// Per-stream header words (int32), see hisparse_meta_layout.
enum HdrWord : int {
  kHdrT = 0,        // LRU clock: number of resolves done
  kHdrStatus = 1,   // status bits of the last resolve
  kHdrPad = 2,      // counters of the last resolve ...
  kHdrRes = 3,
  kHdrHit = 4,
  kHdrMiss = 5,
  kHdrEvict = 6,
  kHdrBytes = 7,
  kHdrTotalMiss = 8,    // int64 running totals since the last reset ...
  kHdrTotalEvict = 10,
  kHdrTotalHit = 12,
  kHdrWords = 16,
};

constexpr int kMaxThreads = 1024;     // resolve workgroup size ceiling
constexpr int kMaxItems = 16;         // items per thread ceiling (C <= 16384)
constexpr int kMaxTopK = 4096;
constexpr int kMaxSlots = 16384;
constexpr int kMaxRequests = 32768;   // the fetch kernel keeps B+1 prefixes in LDS
constexpr size_t kMaxLdsBytes = 163840;   // gfx950: 160 KiB of LDS per workgroup
constexpr int kFetchThreads = 256;
constexpr int kFetchStreamSlices = 8;  // below this many streams the fetch grid is sliced per stream


// Byte layout of the metadata buffer (mirrors hisparse_meta_layout).
inline hisparse_meta_layout meta_layout(const hisparse_config& c) {
  hisparse_meta_layout m{};
  m.status = 0;
  m.stream_base = 256;
  m.hdr = 0;
  m.pos2slot = 256;
  m.slot2pos = m.pos2slot + align256(4 * (size_t)c.max_positions);
  m.last_use = m.slot2pos + align256(4 * (size_t)c.cache_slots);
  m.lru_order = m.last_use + align256(4 * (size_t)c.cache_slots);
  m.evict_log = m.lru_order + align256(4 * (size_t)c.cache_slots);
  m.miss_list = m.evict_log + align256(8 * (size_t)c.top_k);
  m.stream_stride = m.miss_list + align256(8 * (size_t)c.top_k);
  m.total_bytes =
      m.stream_base + (size_t)c.num_layers * (size_t)c.num_requests * m.stream_stride;
  return m;
}

// Launch shape of the resolve kernel: `threads` threads with `items` LRU-order
// entries each cover max(k, C); `sel_items` selections each cover k.
struct ResolveShape {
  int items;
  int threads;
  size_t lds_bytes;
  int sel_items;
};

// Everything a kernel needs to address one layer's streams.
struct StreamView {
  uint8_t* meta;          // metadata buffer base
  uint8_t* cache;         // device cache base
  uint8_t* const* host;   // device array [L*B] of host-history pointers
  int64_t stream_stride;  // bytes between stream blocks
  int64_t off_hdr, off_pos2slot, off_slot2pos, off_last_use, off_order, off_evict,
      off_miss;
  int64_t stream_base;
  int64_t row_bytes;
  int32_t B, L, C, R, k;
  int32_t l_cap;
  uint32_t flags;
  uint32_t r_magic;    // floor(2^32 / R) (2^32 - 1 for R <= 1): fast p mod R
  uint32_t cpr_magic;  // the same for row_bytes / 16 (16-byte chunks per row)
  int32_t fuse_fetch;  // resolve workgroups copy their own misses
};

inline uint32_t div_magic(uint32_t d) {
  return d <= 1 ? 0xFFFFFFFFu : (uint32_t)((uint64_t(1) << 32) / d);
}

// multi_entries > 0: rows of that many entries from several query tokens
// (repeated positions allowed), see hisparse_resolve_multi.
ResolveShape resolve_shape(int k, int C, bool debug_validate, int multi_entries = 0);

// Kernel launchers (hisparse_kernels.hip).  All are asynchronous on `s`.
hipError_t launch_init(const StreamView& v, hipStream_t s, int layer, int request,
                       bool clear_status);
// ev0 / ev1 (optional): events taking the start and end time of the kernel
// itself (eager calls only, not under capture).
hipError_t launch_resolve(const StreamView& v, hipStream_t s, int layer, const int32_t* sel,
                          const int32_t* ctx_len, int32_t* out, int32_t* sel_copy,
                          int multi_entries = 0, const uint8_t* app_rows = nullptr,
                          const int32_t* app_pos = nullptr, hipEvent_t ev0 = nullptr,
                          hipEvent_t ev1 = nullptr);
hipError_t launch_fetch(const StreamView& v, hipStream_t s, int layer, int grid_x,
                        hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_prefetch_join(const StreamView& v, hipStream_t s, const int32_t* sel,
                                const int32_t* sel_copy, const int32_t* pf_out, int32_t* out);
hipError_t launch_load_window(const StreamView& v, hipStream_t s, int layer,
                              const int32_t* ctx_len);
hipError_t launch_append(const StreamView& v, hipStream_t s, int layer, const uint8_t* rows,
                         const int32_t* pos);
hipError_t launch_probe_host_read(hipStream_t s, const void* host, void* dev, size_t bytes,
                                  int workgroups);

}  // namespace hsp
