// Internal declarations shared by the host runtime and the gfx950 kernels of
// libhisparse.  Not part of the C ABI (see include/hisparse.h).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "hisparse.h"

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

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

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

// Launch shape of the resolve kernel: `items` entries per thread (a power of
// two) and `threads` threads cover max(k, C) entries.
struct ResolveShape {
  int items;
  int threads;
  size_t lds_bytes;
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
hipError_t launch_resolve(const StreamView& v, hipStream_t s, int layer, const int32_t* sel,
                          const int32_t* ctx_len, int32_t* out, int32_t* sel_copy,
                          int multi_entries = 0, const uint8_t* app_rows = nullptr,
                          const int32_t* app_pos = nullptr);
hipError_t launch_fetch(const StreamView& v, hipStream_t s, int layer, int grid_x);
hipError_t launch_prefetch_join(const StreamView& v, hipStream_t s, const int32_t* sel,
                                const int32_t* sel_copy, const int32_t* pf_out, int32_t* out);
hipError_t launch_load_window(const StreamView& v, hipStream_t s, int layer,
                              const int32_t* ctx_len);
hipError_t launch_append(const StreamView& v, hipStream_t s, int layer, const uint8_t* rows,
                         const int32_t* pos);
hipError_t launch_probe_host_read(hipStream_t s, const void* host, void* dev, size_t bytes,
                                  int workgroups);

// ---- top-k selection over indexer scores ---------------------------------------
constexpr int kTopkChunk = 4096;          // positions per workgroup of the scan kernels
constexpr int kTopkThreads = 256;         // threads of the scan kernels
constexpr int kTopkBins = 4096;           // level-1 histogram: top 12 key bits
constexpr int kTopkCntStride = 64;        // candidate counter words per row
constexpr int kTopkMaxRows = 65535;       // grid.y of the scan kernels
constexpr int64_t kTopkMaxLen = (int64_t(1) << 31) - kTopkChunk;

struct TopkArgs {
  const float* scores;    // [rows][row_stride]
  int64_t row_stride;     // floats between rows (multiple of 4)
  int64_t max_len;        // positions per row the workspace is sized for
  const int32_t* ctx_len; // [rows]: eligible positions [0, ctx), clamped
  int32_t k;
  int32_t rows;
  uint32_t* hist;         // [rows][4096] top-12-bit counts, zero between calls
  uint32_t* hist2;        // [rows][4096] next-12-bit counts of the candidates, zero between calls
  uint32_t* cnt;          // [rows][64] counters and the threshold, zero between calls
  uint32_t* bitmap;       // [rows][bm_words]
  int64_t bm_words;
  uint32_t* cand;         // [rows][max_len][2]: (key, position)
  int32_t* out;           // [rows][k]
};

struct TopkLayout {
  size_t hist, hist2, cnt, bitmap, cand, total;  // byte offsets in the workspace
  int64_t bm_words;
};

TopkLayout topk_layout(int rows, int64_t max_len);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// ---- sparse MLA decode attention over the slot map ----------------------------
constexpr int kMlaDqk = 576;        // latent 512 + rope 64 (bf16)
constexpr int kMlaDv = 512;         // value = the latent part
constexpr int kMlaHB = 16;          // heads per workgroup
constexpr int kMlaWaves = 4;
constexpr int kMlaThreads = 64 * kMlaWaves;
constexpr int kMlaMaxSplits = 256;

struct MlaArgs {
  const uint8_t* cache;       // slot rows of (request 0, layer)
  int64_t stream_bytes;       // bytes between consecutive requests' slot rows
  int64_t row_bytes;          // bytes per slot
  int32_t slots_total;        // C + R
  int32_t T;                  // token rows per slot
  int32_t k;                  // slot-map entries per attention row
  int32_t B;                  // attention rows (requests x query tokens)
  int32_t Qn;                 // attention rows per request: row r reads stream r / Qn
  int32_t H, HBn, S;          // heads, head blocks, splits of the token rows
  int32_t rows_per_split;     // multiple of 64
  float scale;
  const __bf16* q;            // [B, H, 576] (B attention rows)
  const int32_t* slots;       // [B, k]
  float* part;                // [B * HBn * S][16][512] partial outputs
  float* part_ml;             // [B * HBn * S][16][2] partial (max, sum)
  float* out;                 // [B, H, 512]
  float* lse;                 // [B, H]
};

struct MlaShape {
  int HBn, S, rows_per_split;
  size_t lds_bytes, part_floats, ml_floats, counters;
};

MlaShape mla_shape(int B, int H, int k, int T);
hipError_t launch_mla(const MlaArgs& a, hipStream_t s, size_t lds_bytes);

}  // namespace hsp
