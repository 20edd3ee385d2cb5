// Internal declarations of the top-k kernels (hisparse_topk.hip) shared with
// the host runtime of libhisparse.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "hisparse_align.h"

namespace hsp {

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

}  // namespace hsp
