// Internal declarations of the sparse MLA attention kernels (hisparse_mla.hip)
// shared with the host runtime of libhisparse.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace hsp {

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
